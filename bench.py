"""Benchmark: wave-index sparse decode attention on one MI355X.

Workload (Llama-3-8B-shaped attention layer at 128K context; RetroInfer summary page,
section 4 evaluates 120K and 1M contexts on Llama3-class models): batch 1, 32 q heads /
8 kv heads, head_dim 128, ctx 131072 bf16 keys/values drawn by the seeded generator;
segments of 8192 tokens with 512 clusters (16 tokens per cluster), 10 k-means rounds;
steady zone 4 sink + 64 local tokens; top 2% of the clusters retrieved.

One step = the whole hot path over one batch of input: the index build of one layer
(segmented k-means + layout) and 64 decode queries.  `value` is decode steps (queries)
per second of that whole job.  Inputs are resident in HBM before timing.  L = 32 layers
live in HBM at distinct addresses; step i rebuilds layer i mod L and its 64 queries visit
the layers round robin, so no decode reuses the 256 MB Infinity Cache.

`--workload` runs one of the method's other workloads instead (16k, 1m, batched: decode
steps/s of the whole job; blocks: the block top-k baseline; shared: the 128K layer with one
retrieval set per kv head; tail: the 128K layer with 4096 tokens decoded after its build; stress: index-build tokens/s of the clustering on 1M heavy-tailed
keys per kv head); the default line is the 128K one.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA

WORKLOAD = dict(workload="llama3-8b-attention-layer-128k", batch=1, q_heads=32, kv_heads=8, head_dim=128,
                ctx=131072, seg_len=8192, clusters_per_seg=512, kmeans_iters=10, n_sink=4, n_local=64,
                topk_frac=0.02, decode_queries_per_step=64, layers=32, seed_data=2, seed_build=1234,
                seed_query=102)
# the other workloads of the method's evaluation (reported with --workload; the default line is
# the 128K one): a small parity-size layer, the 1M-token layer, a ragged batch of 16 sequences
# of 64K..128K tokens, the block top-k baseline on the 128K layer, and the clustering alone on
# 1M heavy-tailed keys per kv head
WORKLOADS = {
    "128k": WORKLOAD,
    "16k": dict(workload="attention-layer-16k", batch=1, q_heads=8, kv_heads=2, head_dim=128, ctx=16384,
                seg_len=8192, clusters_per_seg=512, kmeans_iters=10, n_sink=4, n_local=64, topk_frac=0.05,
                decode_queries_per_step=64, layers=64, seed_data=1, seed_build=1234, seed_query=101),
    "1m": dict(workload="llama3-8b-attention-layer-1m", batch=1, q_heads=32, kv_heads=8, head_dim=128,
               ctx=1048576, seg_len=16384, clusters_per_seg=1024, kmeans_iters=10, n_sink=4, n_local=512,
               topk_frac=0.018, decode_queries_per_step=32, layers=2, seed_data=3, seed_build=1234,
               seed_query=103),
    "batched": dict(workload="batched-decode-16-ragged-64k-128k", batch=16, q_heads=32, kv_heads=8, head_dim=128,
                    ctx=[65536, 131072], seg_len=8192, clusters_per_seg=512, kmeans_iters=10, n_sink=4,
                    n_local=64, topk_frac=0.02, decode_queries_per_step=64, layers=2, seed_data=4,
                    seed_build=1234, seed_query=104),
    # the block top-k baseline on the 128K layer: contiguous blocks of 16 tokens instead of the
    # k-means clusters and no estimation zone (a same-hardware comparison point)
    "blocks": dict(WORKLOAD, workload="block-topk-baseline-128k", blocks=True, kmeans_iters=0),
    # the 128K layer with half a segment of tokens decoded after its build (wave_attn_decode_tail)
    "tail": dict(WORKLOAD, workload="llama3-8b-attention-layer-128k-plus-4096-decoded", tail=4096),
    # the 128K layer with one retrieval set per kv head (wave_attn_decode_shared)
    "shared": dict(WORKLOAD, workload="llama3-8b-attention-layer-128k-shared-selection", shared=True),
    # the 1M layer with bf16 value sums (the estimation zone reads half the bytes)
    "1m-bf16-sums": dict(workload="llama3-8b-attention-layer-1m-bf16-value-sums", batch=1, q_heads=32, kv_heads=8,
                         head_dim=128, ctx=1048576, seg_len=16384, clusters_per_seg=1024, kmeans_iters=10, n_sink=4,
                         n_local=512, topk_frac=0.018, decode_queries_per_step=32, layers=2, seed_data=3,
                         seed_build=1234, seed_query=103, value_sums="bf16"),
    "stress": dict(workload="index-build-1m-keys-student-t", batch=1, q_heads=8, kv_heads=8, head_dim=128,
                   ctx=1048576, seg_len=8192, clusters_per_seg=512, kmeans_iters=10, heavy_tailed=True,
                   n_sink=4, n_local=64, topk_frac=0.02, decode_queries_per_step=0, layers=1, seed_data=5,
                   seed_build=1234, seed_query=105),
}


def num_clusters(n, seg, ks):
    """Clusters of a sequence of n tokens: K_s per full segment, ceil(L K_s / L_s) for a short last one."""
    nseg = -(-n // seg)
    last = n - (nseg - 1) * seg
    return (nseg - 1) * ks + (ks if last >= seg else -(-last * ks // seg))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", choices=sorted(WORKLOADS), default="128k",
                   help="workload of the line (default: the 128K layer, the headline one)")
    p.add_argument("--layers", type=int, default=None, help="layer indexes in HBM (default: the workload's)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="the headline line without the 1m, batched and stress workloads' figures")
    p.add_argument("--cpu-seconds", type=float, default=20.0, help="budget of the oracle timing sample")
    p.add_argument("--cpu-single-thread", action="store_true",
                   help="(run by the CPU baseline in a child process with OMP_NUM_THREADS=1) time one k-means "
                        "unit, one index layout and two decode queries of the 128K layer and print them")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a device copy of 1 GiB (scale of the HBM byte counters)")
    p.add_argument("--eager", action="store_true",
                   help="time eager launches instead of graph replays (for counter collection)")
    p.add_argument("--summarize-trace", metavar="DIR",
                   help="print the per-kernel table of a rocprofv3 --kernel-trace --stats csv run and exit")
    p.add_argument("--summarize-traffic", nargs=5, metavar=("KERNEL", "FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR",
                                                            "CAL_WRITE_DIR"),
                   help="print HBM bytes per launch of KERNEL from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE csv "
                        "runs of the benchmark and of --calibrate-copy, and exit")
    p.add_argument("--summarize-mfma", nargs=2, metavar=("KERNEL", "DIR"),
                   help="print the MFMA utilisation of KERNEL from a rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES "
                        "GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_BF16 csv run, and exit")
    p.add_argument("--command", default="", help="command line recorded in a summary")
    p.add_argument("--accuracy", action="store_true",
                   help="only measure the error of the wave attention against dense attention over a grid of "
                        "budgets (top-k fraction, local window, clusters per segment) on the 128K layer")
    return p.parse_args()


def source_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(kernel, sha, tag="128k"):
    """HBM bytes per launch from a committed rocprofv3 counter summary of workload `tag`, if it matches the
    source."""
    kernel = {"k_sort": "k_sort_radix"}.get(kernel, kernel)  # the launch name of the LDS radix sort
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.txt" % (kernel, tag))
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha") != sha:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _csv_rows(d, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)):
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit("no *%s under %s" % (suffix, d))
    return rows


def _short(name):
    """wave::k_attend<4>(...) -> k_attend<4>; other kernels keep 60 characters."""
    base = name.split("(")[0].replace("void ", "").strip()
    return base.split("::")[-1] if "wave::" in base else base[:60]


def summarize_trace(d, command):
    rows = _csv_rows(d, "kernel_stats.csv")
    out = ["# rocprofv3 kernel statistics", "command: %s" % command, "",
           "%-28s %8s %12s %12s %12s %12s %7s" % ("kernel", "calls", "total_us", "avg_us", "min_us", "max_us", "pct")]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        out.append("%-28s %8d %12.1f %12.2f %12.2f %12.2f %7.2f" % (
            _short(r["Name"]), int(r["Calls"]), float(r["TotalDurationNs"]) / 1e3, float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    print("\n".join(out))


# kernels launched under one name: the assign runs k_assign_lds up to 512 clusters a segment,
# k_assign<true> above
_KERNELS_OF = {"k_assign": ("k_assign", "k_assign_lds")}


def _is_kernel(name, kernel):
    return _short(name).split("<")[0] in _KERNELS_OF.get(kernel, (kernel,))


def _counter_per_dispatch(d, counter, kernel=None):
    """Per-dispatch values of one counter; the kernel's dispatches, or the largest one."""
    vals = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        key = (r["Dispatch_Id"], r["Kernel_Name"])
        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    if kernel is None:
        return [max(vals.values())]
    return [v for (_, n), v in vals.items() if _is_kernel(n, kernel)]


def summarize_traffic(kernel, fdir, wdir, cfdir, cwdir, command):
    n_cal = 1 << 30
    cf = _counter_per_dispatch(cfdir, "FETCH_SIZE")[0] * 1024.0
    cw = _counter_per_dispatch(cwdir, "WRITE_SIZE")[0] * 1024.0
    f = _counter_per_dispatch(fdir, "FETCH_SIZE", kernel)
    w = _counter_per_dispatch(wdir, "WRITE_SIZE", kernel)
    if not f or not w:
        raise SystemExit("no dispatch of %s in the counter runs" % kernel)
    fs, ws_ = n_cal / cf, n_cal / cw
    fb = sum(f) / len(f) * 1024.0 * fs
    wb = sum(w) / len(w) * 1024.0 * ws_
    sha = source_sha(SOURCES)
    print("\n".join([
        "# HBM traffic of %s per launch (rocprofv3 --pmc, TCC counters in KiB per dispatch)" % kernel,
        "command: %s" % command,
        "calibration: a device copy of %d bytes read FETCH_SIZE %.0f B (scale %.4f), WRITE_SIZE %.0f B (scale %.4f)"
        % (n_cal, cf, fs, cw, ws_),
        "dispatches: %d fetch, %d write" % (len(f), len(w)),
        "fetch_bytes_per_launch: %.0f" % fb,
        "write_bytes_per_launch: %.0f" % wb,
        "hbm_bytes_per_launch: %.0f" % (fb + wb),
        "source_sha: %s" % sha]))


def summarize_mfma(kernel, d, command):
    """MFMA utilisation of a kernel's dispatches. On this GPU rocprofv3 reports one row per dispatch and
    counter, summed over the chip: GRBM_GUI_ACTIVE over its 8 XCDs (so per-XCD cycles are a
    dispatch's clock cycles, which against the dispatch's duration give the clock it ran at) and
    SQ_VALU_MFMA_BUSY_CYCLES over its 1024 SIMDs. Busy fraction = busy cycles per SIMD over
    per-XCD cycles; bf16 flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512."""
    per = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        if not _is_kernel(r["Kernel_Name"], kernel):
            continue
        e = per.setdefault(r["Dispatch_Id"], {})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        e["ns"] = float(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    if not per:
        raise SystemExit("no dispatch of %s in %s" % (kernel, d))
    xcds, simds = 8, 256 * 4
    n = len(per)
    mean = lambda key: sum(e.get(key, 0.0) for e in per.values()) / n
    busy, gui, ns = mean("SQ_VALU_MFMA_BUSY_CYCLES"), mean("GRBM_GUI_ACTIVE") / xcds, mean("ns")
    flops = mean("SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512.0
    frac = busy / simds / gui
    fpc = flops / gui
    print("\n".join([
        "# MFMA utilisation of %s (rocprofv3 --pmc, one dispatch at a time)" % kernel,
        "command: %s" % command,
        "dispatches: %d, mean duration %.1f us (profiled)" % (n, ns / 1000.0),
        "GRBM_GUI_ACTIVE per dispatch: %.0f summed over %d XCDs = %.0f cycles per XCD (clock %.3f GHz)"
        % (gui * xcds, xcds, gui, gui / ns),
        "SQ_VALU_MFMA_BUSY_CYCLES per dispatch: %.0f summed over %d SIMDs = %.0f per SIMD" % (busy, simds, busy / simds),
        "mfma_busy_fraction (per SIMD, of the dispatch's cycles): %.4f" % frac,
        "bf16 MFMA flops per dispatch (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512): %.4g" % flops,
        "bf16 MFMA flops per cycle: %.0f of 1048576 (256 CUs x 4096) = %.4f" % (fpc, fpc / 1048576.0),
        "achieved over the profiled duration: %.1f TFLOP/s = %.4f of the 2.5 PFLOP/s peak (at 2.4 GHz)"
        % (flops / ns / 1e3, flops / ns / 1e3 / BF16_PEAK_TFLOPS)]))


SOURCES = ["retrieval_sparse_attention_amd/csrc/decode.hip", "retrieval_sparse_attention_amd/csrc/build.hip",
           "retrieval_sparse_attention_amd/csrc/common.h", "retrieval_sparse_attention_amd/csrc/internal.h",
           "retrieval_sparse_attention_amd/csrc/wave_attn.hip"]


def accuracy(dev):
    """Error of the wave attention and of two baselines against dense softmax attention.

    The 128K layer's generator (drifting Gaussian mixture keys and values, queries near a
    uniformly drawn key), 16 queries per q head. For each clusters_per_seg, topk_frac and
    n_local: relative L2 error |o - o_dense| / |o_dense| per (query, q head) (mean, 90th
    percentile, maximum) and the share of tokens read exactly (retrieved plus steady), for
    the wave attention over the k-means index, the same with one selection per kv head
    (wave-shared), the same selection without the estimation zone, and the block top-k
    baseline (contiguous blocks, no estimation). The dense
    reference is float32 softmax attention in PyTorch over all N keys.
    """
    import numpy as np
    import torch

    import retrieval_sparse_attention_amd as rsa
    import synth

    W = WORKLOAD
    B, H, G, N, seg = 1, W["q_heads"], W["kv_heads"], W["ctx"], W["seg_len"]
    ns, iters, nq = W["n_sink"], W["kmeans_iters"], 16
    ctx = np.array([N], np.int64)
    print("generating inputs", file=sys.stderr, flush=True)
    K, V, _ = synth.kv(W["seed_data"], B, G, ctx, seg)
    q, _ = synth.queries(W["seed_query"], nq, B, H, G, ctx, K)
    Kd = torch.from_numpy(K.view(np.int16)).to(dev).view(torch.bfloat16)
    Vd = torch.from_numpy(V.view(np.int16)).to(dev).view(torch.bfloat16)
    qd = torch.from_numpy(q.view(np.int16)).to(dev).view(torch.bfloat16)  # [nq, 1, H, 128]
    tau = 1.0 / math.sqrt(128.0)
    Kf = Kd.view(G, N, 128).float()
    Vf = Vd.view(G, N, 128).float()
    qf = qd.view(nq, G, H // G, 128).float()
    ref = torch.empty((nq, G, H // G, 128), dtype=torch.float32, device=dev)
    for g in range(G):
        s = torch.matmul(qf[:, g].reshape(-1, 128), Kf[g].t().contiguous()) * tau  # [nq * H/G, N]
        ref[:, g] = torch.matmul(torch.softmax(s, dim=1), Vf[g]).view(nq, H // G, 128)
    ref = ref.view(nq, H, 128)
    rows = []
    # the wave attention over the k-means index at every budget; for a local window of 64 also
    # the same selection without the estimation zone, and the block top-k baseline (contiguous
    # blocks, no estimation)
    runs = [("wave", False, True, nl) for nl in (0, 64, 512)] + [("wave-shared", False, True, 64),
                                                                  ("kmeans-topk-only", False, False, 64),
                                                                  ("block-topk", True, False, 64)]
    for ks in (256, 512, 1024):
        kidx = rsa.wave_index_build(Kd, Vd, G, [N], seg, ks, iters, W["seed_build"])
        bidx = rsa.wave_index_build_blocks(Kd, Vd, G, [N], seg, ks)
        for method, blocks, estimate, nl in runs:
            idx = bidx if blocks else kidx
            sizes = idx.arrays["sizes"].cpu().numpy()
            C = sizes.size // G
            for frac in (0.005, 0.01, 0.02, 0.05, 0.1):
                err, exact = [], []
                for t in range(nq):
                    o, ids, _ = rsa.wave_attn_decode(idx, qd[t], ns, nl, frac, estimate=estimate,
                                                     shared=method == "wave-shared")
                    e = (o[0] - ref[t]).norm(dim=1) / ref[t].norm(dim=1)
                    err.append(e.cpu().numpy())
                    ih = ids[0].cpu().numpy()
                    for h in range(H):
                        sel = ih[h][ih[h] >= 0]
                        exact.append((sizes[(h * G // H) * C + sel].sum() + ns + nl) / N)
                err = np.concatenate(err)
                rows.append({"method": method, "clusters_per_seg": ks, "n_local": nl, "topk_frac": frac,
                             "rel_err_mean": round(float(err.mean()), 5),
                             "rel_err_p90": round(float(np.quantile(err, 0.9)), 5),
                             "rel_err_max": round(float(err.max()), 5),
                             "exact_token_share": round(float(np.mean(exact)), 4)})
                print("%-16s K_s %4d n_local %3d frac %.3f: rel err mean %.4f max %.4f, exact tokens %.3f" % (
                    method, ks, nl, frac, rows[-1]["rel_err_mean"], rows[-1]["rel_err_max"],
                    rows[-1]["exact_token_share"]), file=sys.stderr, flush=True)
        del kidx, bidx
    print(json.dumps({"metric": "relative L2 error against dense attention (wave attention and baselines)",
                      "workload": W["workload"], "queries_per_head": nq, "q_heads": H, "n_sink": ns,
                      "data": "synthetic", "reference": "float32 dense softmax attention (PyTorch)", "rows": rows}))


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.command)
        return
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, command=args.command)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma, command=args.command)
        return
    if args.cpu_single_thread:
        cpu_single_thread_sample()
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU: this build has no multi-GPU path (the kv-head sharding it "
              "would use is described in DESIGN.md); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import retrieval_sparse_attention_amd as rsa
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        n = 1 << 30
        # an elementwise kernel that reads and writes n bytes once (fp32 negation)
        x = torch.ones(n // 4, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(x, out=y)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n, "launches": 3}))
        return

    if args.accuracy:
        accuracy(dev)
        return

    W = dict(WORKLOADS[args.workload])
    if args.layers is not None:
        W["layers"] = args.layers
    headline = args.workload == "128k"
    result, (K, V, ctx, q) = measure(W, args.steps, args.warmup, args.eager, headline, dev)
    if headline and not args.no_extra:
        # the method's other evaluated shapes, each from its own inputs and indexes, on fewer steps
        # (decode per query, achieved bandwidth of the decode, index build, k_assign's MFMA rate)
        extra = {}
        for name, st in (("1m", 4), ("1m-bf16-sums", 4), ("batched", 4), ("stress", 3)):
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            r, _ = measure(dict(WORKLOADS[name]), st, 1, args.eager, False, dev)
            extra[name] = workload_summary(r)
        result["workloads"] = extra
        torch.cuda.empty_cache()
        result["append"] = measure_append(W, dev)
        torch.cuda.empty_cache()
        result["stochastic_topk"] = {n: measure_stochastic(dict(WORKLOADS[n]), dev) for n in ("128k", "1m")}
        torch.cuda.empty_cache()
    if headline and not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(W, K, V, ctx, q, args.cpu_seconds)
    print(json.dumps(result))


def measure_append(W, dev, reps=10):
    """In-place growth of the 128K layer's index (wave_index_append) against a rebuild over
    the longer context: one appended segment of seg_len tokens per kv head, and one token
    appended into a half-full last segment (which re-clusters that whole segment)."""
    import numpy as np
    import torch

    import retrieval_sparse_attention_amd as rsa
    import synth
    G, seg, K_s, iters, seed = W["kv_heads"], W["seg_len"], W["clusters_per_seg"], W["kmeans_iters"], W["seed_build"]
    N0 = W["ctx"]
    N1 = N0 + seg
    cap = N1 // seg + 1
    K, V, _ = synth.kv(W["seed_data"], 1, G, np.array([N1 + seg], np.int64), seg)
    Nf = N1 + seg

    def rows(lo, hi):
        return np.concatenate([np.arange(g * Nf + lo, g * Nf + hi) for g in range(G)])

    def dev_rows(lo, hi):
        r = rows(lo, hi)
        return (torch.from_numpy(K[r].view(np.int16)).to(dev).view(torch.bfloat16),
                torch.from_numpy(V[r].view(np.int16)).to(dev).view(torch.bfloat16))

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn, before=None):
        ts = []
        for _ in range(reps):
            if before:
                before()
            torch.cuda.synchronize()
            ev[0].record()
            fn()
            ev[1].record()
            torch.cuda.synchronize()
            ts.append(ev[0].elapsed_time(ev[1]))
        return float(np.median(ts))

    K0, V0 = dev_rows(0, N0)
    ix = rsa.wave_index_build(K0, V0, G, [N0], seg, K_s, iters, seed, cap_segs=cap)
    kn, vn = dev_rows(N0, N1)
    ws = torch.empty(rsa.wave_index_append_plan(ix, [N1]), dtype=torch.uint8, device=dev)
    t_seg = timed(lambda: rsa.wave_index_append(ix, kn, vn, [N1], iters, seed, ws=ws), before=lambda: ix.set_ctx([N0]))
    K1, V1 = dev_rows(0, N1)
    ix1 = rsa.wave_index_build(K1, V1, G, [N1], seg, K_s, iters, seed)
    bws = torch.empty(rsa.wave_index_plan(G, [N1], seg, K_s)["build_ws_bytes"], dtype=torch.uint8, device=dev)
    t_re = timed(lambda: rsa.wave_index_build(K1, V1, G, [N1], seg, K_s, iters, seed, index=ix1, ws=bws))
    # one token into a half-full last segment
    Nh = N0 + seg // 2
    Kh, Vh = dev_rows(0, Nh)
    ixh = rsa.wave_index_build(Kh, Vh, G, [Nh], seg, K_s, iters, seed, cap_segs=cap)
    k1, v1 = dev_rows(Nh, Nh + 1)
    ws1 = torch.empty(rsa.wave_index_append_plan(ixh, [Nh + 1]), dtype=torch.uint8, device=dev)
    t_tok = timed(lambda: rsa.wave_index_append(ixh, k1, v1, [Nh + 1], iters, seed, ws=ws1),
                  before=lambda: ixh.set_ctx([Nh]))
    torch.cuda.synchronize()
    return {"workload": "llama3-8b-attention-layer-128k-append", "kv_heads": G, "seg_len": seg,
            "ms_append_one_segment": round(t_seg, 3), "append_tokens_per_s": round(G * seg / (t_seg / 1000.0)),
            "ms_rebuild_%d" % N1: round(t_re, 3), "rebuild_over_append": round(t_re / t_seg, 2),
            "ms_append_one_token_into_half_segment": round(t_tok, 3), "reps": reps, "timing": "median of reps"}


def measure_stochastic(W, dev, nq=16, seed=2024):
    """The stochastic radix top-k variant (wave_attn_decode_stochastic) against the exact selection
    on one layer of workload W: recall of the exact ids, relative L2 error of both against dense
    float32 softmax attention, the top-k kernel's average time (dispatch-recorded events) and
    the decode call's time (event-timed eager calls), over nq queries."""
    import numpy as np
    import torch

    import retrieval_sparse_attention_amd as rsa
    import synth
    G, H, N, seg, K_s = W["kv_heads"], W["q_heads"], W["ctx"], W["seg_len"], W["clusters_per_seg"]
    ns, nl, frac = W["n_sink"], W["n_local"], W["topk_frac"]
    ctx = np.array([N], np.int64)
    K, V, _ = synth.kv(W["seed_data"], 1, G, ctx, seg)
    q, _ = synth.queries(W["seed_query"], nq, 1, H, G, ctx, K)
    Kd = torch.from_numpy(K.view(np.int16)).to(dev).view(torch.bfloat16)
    Vd = torch.from_numpy(V.view(np.int16)).to(dev).view(torch.bfloat16)
    qd = torch.from_numpy(q.view(np.int16)).to(dev).view(torch.bfloat16)
    del K, V
    ix = rsa.wave_index_build(Kd, Vd, G, [N], seg, K_s, W["kmeans_iters"], W["seed_build"])
    tau = 1.0 / math.sqrt(128.0)
    ref = torch.empty((nq, H, 128), dtype=torch.float32, device=dev)
    for g in range(G):
        Kg, Vg = Kd[g * N:(g + 1) * N].float(), Vd[g * N:(g + 1) * N].float()
        qg = qd[:, 0, g * (H // G):(g + 1) * (H // G)].float().reshape(-1, 128)
        s = torch.matmul(qg, Kg.t().contiguous()) * tau
        ref[:, g * (H // G):(g + 1) * (H // G)] = torch.matmul(torch.softmax(s, dim=1), Vg).view(nq, H // G, 128)
        del Kg, Vg, s
    k_max, wsb = rsa.wave_attn_decode_plan(ix, H, ns, nl, frac)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def run(passes):
        call = (lambda t: rsa.wave_attn_decode(ix, qd[t], ns, nl, frac, ws=ws)) if passes == 0 else (
            lambda t: rsa.wave_attn_decode_stochastic(ix, qd[t], ns, nl, frac, passes, seed + t, ws=ws))
        outs = [call(t) for t in range(nq)]  # warm
        torch.cuda.synchronize()
        ev[0].record()
        for t in range(nq):
            call(t)
        ev[1].record()
        torch.cuda.synchronize()
        us = 1000.0 * ev[0].elapsed_time(ev[1]) / nq
        rsa.wave_profiler_enable(True)
        for t in range(nq):
            call(t)
        torch.cuda.synchronize()
        rsa.wave_profiler_enable(False)
        prof = rsa.wave_profiler_read()
        name = "k_topk" if passes == 0 else "k_topk_sto"
        tk = 1000.0 * prof[name][1] / prof[name][0]
        ids = [o[1].cpu().numpy() for o in outs]
        err = torch.cat([((o[0][0] - ref[t]).norm(dim=1) / ref[t].norm(dim=1)) for t, o in enumerate(outs)])
        return ids, err.cpu().numpy(), us, tk

    ex_ids, ex_err, ex_us, ex_tk = run(0)
    out = {"workload": W["workload"], "queries": nq, "k_max": k_max,
           "exact": {"rel_err_mean": round(float(ex_err.mean()), 5), "decode_us_per_query": round(ex_us, 2),
                     "topk_us": round(ex_tk, 2)}}
    for passes in (1, 2, 3):
        ids, err, us, tk = run(passes)
        hit = tot = 0
        for a, e in zip(ids, ex_ids):
            for h in range(H):
                sa_, se = a[0, h], e[0, h]
                sa_, se = set(sa_[sa_ >= 0].tolist()), set(se[se >= 0].tolist())
                hit += len(sa_ & se)
                tot += len(se)
        out["passes_%d" % passes] = {"recall": round(hit / max(tot, 1), 4), "rel_err_mean": round(float(err.mean()), 5),
                                     "rel_err_max": round(float(err.max()), 5), "decode_us_per_query": round(us, 2),
                                     "topk_us": round(tk, 2)}
        print("stochastic top-k %s passes %d: recall %.4f, rel err %.5f (exact %.5f), top-k %.1f us (exact %.1f)"
              % (W["workload"], passes, hit / max(tot, 1), err.mean(), ex_err.mean(), tk, ex_tk), file=sys.stderr,
              flush=True)
    del ix, Kd, Vd, ref
    return out


def workload_summary(r):
    """The figures of another workload's line that the headline line carries."""
    ka = r["kernel_roofline"].get("k_assign", {})
    out = {"metric": r["metric"], "value": r["value"], "unit": r["unit"], "steps": r["steps"],
           "ms_per_step": r["ms_per_step"], "config": r["config"],
           "decode_only_us_per_query": r["decode_only_us_per_query"],
           "decode_only_effective_GBs": r["decode_only_effective_GBs"],
           "decode_only_frac_of_hbm_peak": (round(r["decode_only_effective_GBs"] / HBM_PEAK_GBS, 4)
                                            if r["decode_only_effective_GBs"] else None),
           "decode_bytes_per_query": r["decode_bytes_per_query"],
           "build_tokens_per_s": r["build_tokens_per_s"],
           "k_assign_TFLOPs": ka.get("achieved_TFLOPs"), "k_assign_frac_of_bf16_peak": ka.get("frac"),
           "kernels": r["kernels"],
           "kernel_roofline": {k: {kk: v[kk] for kk in ("frac", "achieved_GBs", "achieved_TFLOPs") if kk in v}
                               for k, v in r["kernel_roofline"].items()}}
    return out


def measure(W, steps, warmup, eager, headline, dev):
    """One workload: inputs, L layer indexes, captured step graphs, the timed steps, the
    decode-only steps, and an eager pass with dispatch-recorded events per kernel. Returns the
    JSON fields of its line and the host inputs (for the oracle's timing)."""
    import numpy as np
    import torch

    import retrieval_sparse_attention_amd as rsa
    import synth

    class _A:  # the step counts of this measurement
        pass
    args = _A()
    args.steps, args.warmup, args.eager = steps, warmup, eager
    B, H, G = W["batch"], W["q_heads"], W["kv_heads"]
    seg, K_s, iters = W["seg_len"], W["clusters_per_seg"], W["kmeans_iters"]
    ns, nl, frac, QPS = W["n_sink"], W["n_local"], W["topk_frac"], W["decode_queries_per_step"]
    L = W["layers"]
    tag = next((k for k, v in WORKLOADS.items() if v["workload"] == W["workload"]), "")  # profiles/ file tag
    blocks = W.get("blocks", False)
    shared = W.get("shared", False)
    if isinstance(W["ctx"], list):  # ragged: N_b ~ U{lo..hi} from the data seed
        ctx = synth.ctx_lengths(W["seed_data"], B, W["ctx"][0], W["ctx"][1])
    else:
        ctx = np.array([W["ctx"]] * B, np.int64)
    N = int(ctx.max())

    print("generating inputs", file=sys.stderr, flush=True)
    K, V, _ = synth.kv(W["seed_data"], B, G, ctx, seg, heavy=W.get("heavy_tailed", False))
    nq = max(QPS, 1) * 4
    q, _ = synth.queries(W["seed_query"], nq, B, H, G, ctx, K)
    Kd0 = torch.from_numpy(K.view(np.int16)).to(dev).view(torch.bfloat16)
    Vd0 = torch.from_numpy(V.view(np.int16)).to(dev).view(torch.bfloat16)
    qd = torch.from_numpy(q.view(np.int16)).to(dev).view(torch.bfloat16)  # [nq, B, H, 128]
    # L layers at distinct addresses (copies of the seeded layer)
    Ks = [Kd0] + [Kd0.clone() for _ in range(L - 1)]
    Vs = [Vd0] + [Vd0.clone() for _ in range(L - 1)]
    z = rsa.wave_index_plan(G, ctx.tolist(), seg, K_s)
    vsums = W.get("value_sums", "f32")
    idxs = [rsa.WaveIndex.allocate(G, ctx.tolist(), seg, K_s, device=dev, value_sums=vsums)[0] for _ in range(L)]
    bws = torch.empty(int(z["build_ws_bytes"]), dtype=torch.uint8, device=dev)
    print("building %d layer indexes" % L, file=sys.stderr, flush=True)
    def build_layer(l):
        if blocks:
            rsa.wave_index_build_blocks(Ks[l], Vs[l], G, ctx.tolist(), seg, K_s, index=idxs[l], ws=bws)
        else:
            rsa.wave_index_build(Ks[l], Vs[l], G, ctx.tolist(), seg, K_s, iters, W["seed_build"], index=idxs[l],
                                 ws=bws)

    for l in range(L):
        build_layer(l)
    torch.cuda.synchronize()
    n_tail = int(W.get("tail", 0))
    if n_tail:
        # the decoded tokens' K/V rows: the generator's next n_tail tokens of each (b, g)
        Kx, Vx, _ = synth.kv(W["seed_data"] + 1, B, G, np.array([n_tail] * B, np.int64), seg)
        k_tail = torch.from_numpy(Kx.view(np.int16)).to(dev).view(torch.bfloat16).view(B, G, n_tail, 128)
        v_tail = torch.from_numpy(Vx.view(np.int16)).to(dev).view(torch.bfloat16).view(B, G, n_tail, 128)
        tail_len = torch.full((B,), n_tail, dtype=torch.int32, device=dev)
        k_max, dwsb = rsa.wave_attn_decode_tail_plan(idxs[0], H, ns, nl, frac, n_tail)
    else:
        k_max, dwsb = rsa.wave_attn_decode_plan(idxs[0], H, ns, nl, frac)
    dws = torch.empty(dwsb, dtype=torch.uint8, device=dev)
    out = torch.empty((B, H, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)

    ids_buf = torch.empty((B, H, max(k_max, 1)), dtype=torch.int32, device=dev)

    def job(step, ids_log=None, build=True):
        """One step: rebuild layer (step mod L), then 64 queries over the layers round robin."""
        l = step % L
        if build:
            build_layer(l)
        for s in range(QPS):
            lay = (step * QPS + s) % L
            qi = (step * QPS + s) % nq
            ids = ids_log[s] if ids_log is not None else ids_buf
            if n_tail:
                rsa.wave_attn_decode_tail(idxs[lay], qd[qi], ns, nl, frac, k_tail, v_tail, tail_len, ws=dws,
                                          out=out, sel_ids=ids, lse=lse)
            else:
                rsa.wave_attn_decode(idxs[lay], qd[qi], ns, nl, frac, ws=dws, out=out, sel_ids=ids, lse=lse,
                                     estimate=not blocks, shared=shared)

    # the step pattern repeats with period P: one captured HIP graph per phase
    P = math.lcm(L, max(1, nq // math.gcd(nq, max(QPS, 1))))
    print("warmup (eager)%s" % ("" if args.eager else " and capture of %d step graphs" % P), file=sys.stderr,
          flush=True)
    for i in range(max(1, args.warmup)):
        job(i)
    torch.cuda.synchronize()
    graphs, dgraphs = [], []
    if not args.eager:
        for ph in range(P):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                job(ph)
            graphs.append(g)
            if QPS > 0:
                g2 = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g2):
                    job(ph, build=False)
                dgraphs.append(g2)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[i % P].replay()
    torch.cuda.synchronize()

    def run(i, build=True):
        if args.eager:
            job(i, build=build)
        else:
            (graphs if build else dgraphs)[i % P].replay()

    # ---- timed region: K whole-job steps (graph replays on the current stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.warmup, args.warmup + args.steps):
        run(i)
    e1.record()
    torch.cuda.synchronize()
    t_plain = e0.elapsed_time(e1)
    print("timed %d steps: %.3f ms" % (args.steps, t_plain), file=sys.stderr, flush=True)
    # decode queries alone (same 64 per step, no build)
    t_dec = None
    if QPS > 0:
        e0.record()
        for i in range(args.warmup, args.warmup + args.steps):
            run(i, build=False)
        e1.record()
        torch.cuda.synchronize()
        t_dec = e0.elapsed_time(e1)

    # ---- the same steps once more, eagerly, with HIP events around every kernel on its
    # launch stream: per-kernel durations for the roofline, and the selected ids
    ids_log = torch.empty((args.steps * QPS, B, H, max(k_max, 1)), dtype=torch.int32, device=dev)
    rsa.wave_profiler_enable(True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.warmup, args.warmup + args.steps):
        job(i, ids_log[(i - args.warmup) * QPS:(i - args.warmup + 1) * QPS])
    e1.record()
    torch.cuda.synchronize()
    rsa.wave_profiler_enable(False)
    prof = rsa.wave_profiler_read()
    t_ms = e0.elapsed_time(e1)

    # ---- algorithmic work per launch (actual sizes of the selected clusters)
    sizes = idxs[0].sizes.cpu().numpy()  # every layer holds the same clustering
    Cb = [num_clusters(int(n), seg, K_s) for n in ctx]
    Ctot = sum(Cb)
    cbase = np.concatenate([[0], np.cumsum([G * c for c in Cb])]).astype(np.int64)
    nq_t = args.steps * QPS
    retrieved_rows, n_sel = 0, 0
    if nq_t > 0:
        ids_h = ids_log[:, :, :, :k_max].cpu().numpy()  # [queries, B, H, k_max]
        for qq in range(nq_t):
            for b in range(B):
                for h in range(H):
                    sel = ids_h[qq, b, h]
                    sel = sel[sel >= 0]
                    n_sel += len(sel)
                    # a shared selection's rows are read once for the kv head's q heads
                    if not shared or h % (H // G) == 0:
                        retrieved_rows += int(sizes[cbase[b] + (h * G // H) * Cb[b] + sel].sum())
    rows_per_dec = retrieved_rows / max(nq_t, 1)
    sel_per_dec = n_sel / max(nq_t, 1)             # clusters selected per decode call, all (b, h)
    # algorithmic HBM bytes per launch: every byte a kernel must read or write once
    steady = ns + nl
    n_est = sum(-(-c // 128) for c in Cb)          # estimation chunks (workgroups) per kv head
    # row workgroups per (b, h), as the library plans them: 176 rows each at the average
    # cluster size if the grid then fits 1024 resident workgroups, else 256
    est_rows = k_max * -(-seg // K_s) + steady
    n_tail_wg = -(-n_tail // 64)                  # appended-token workgroups per kv head
    P = -(-est_rows // 176)
    if B * H * P + G * n_est > 1024:
        P = -(-est_rows // 256)
    P = max(1, min(4096, P))
    part = 132 * 4                                # one partial softmax state
    rows = G * int(ctx.sum())                     # index rows
    score_bytes = (G * Ctot * (128 * 2 + 4)       # bf16 centroid rows + sizes
                   + B * H * 128 * 2              # q
                   + H * Ctot * 8                 # rank keys + sortable keys out
                   + B * G * n_tail * 2 * 128 * 2  # appended tokens' K, V (their workgroups run in this grid)
                   + (B * H * n_tail_wg * part if n_tail else 0))
    sel_words = H * sum(-(-c // 32) for c in Cb)  # selection bitmap words (all q heads)
    topk_bytes = (H * Ctot * 4 + G * Ctot * 8     # sortable keys; sizes + offsets
                  + sel_per_dec * (4 + 8 + 4)     # ids, spans, member prefix out
                  + sel_words * 4                 # the selection bitmaps out (for the estimation role)
                  + B * H * steady * 8)           # steady rows: cluster ids in, corrections out
    attend_bytes = (rows_per_dec * (2 * 128 * 2 + 4)         # K, V and perm of the retrieved rows
                    + B * G * steady * (2 * 128 * 2 + 4)      # steady rows (a kv head's): K, V, inv_perm
                    + B * H * steady * 4                      # their corrections per q head
                    + sel_per_dec * 12                        # window metadata
                    + B * H * 128 * 2 + B * H * P * part)     # q, row partials out
    if not blocks:
        vs_read = 128 * 2 if vsums in ("bf16", "both") else 128 * 4
        attend_bytes += (G * Ctot * (vs_read + 4)             # estimation: value sums + sizes
                         + H * Ctot * 4 + sel_words * 4       # estimation: rank keys, selection bitmaps
                         + H * n_est * part)                  # estimation partials out
    merge_bytes = (B * H * P * part + (0 if blocks else H * n_est * part) + B * H * n_tail_wg * part
                   + B * H * (128 * 4 + 4))
    step_bytes = score_bytes + topk_bytes + attend_bytes + merge_bytes
    # per launch (one k-means round): every unit's tokens against its own clusters
    tok_clu = 0
    for n in ctx:
        n = int(n)
        nseg = -(-n // seg)
        for si in range(nseg):
            ls = min(seg, n - si * seg)
            tok_clu += ls * (K_s if ls >= seg else -(-ls * K_s // seg))
    assign_flops = 2.0 * 128 * G * tok_clu
    assign_bytes = rows * (128 * 2 + 4) + G * Ctot * (128 * 2 + 4)
    vs_write = {"f32": 128 * 4, "bf16": 128 * 2, "both": 128 * 6}[vsums]
    final_update = rows * (4 * 128 * 2 + 3 * 4) + G * Ctot * (128 * 4 + vs_write + 128 * 2 + 4)
    update_bytes = (final_update if blocks else
                    ((iters - 1) * (rows * (128 * 2 + 4) + G * Ctot * (128 * 4 + 128 * 2 + 4)) + final_update) / iters)
    sort_bytes = rows * 12 + G * Ctot * 8
    init_bytes = G * Ctot * (128 * 2 + 128 * 4 + 128 * 2 + 4)
    hbm_bytes = {"k_score": score_bytes, "k_topk": topk_bytes, "k_attend": attend_bytes, "k_merge": merge_bytes,
                 "k_update": update_bytes, "k_sort": sort_bytes, "k_init": init_bytes, "k_block_assign": rows * 4}

    kern = {}
    for name, (cnt, ms) in prof.items():
        kern[name] = {"launches": cnt, "avg_us": 1000.0 * ms / cnt, "total_ms": ms}
    # committed counter summaries exist for the 128K and 1M workloads (profiles/traffic_<kernel>_<tag>.txt)
    sha = source_sha(SOURCES)
    dom = max((k for k in kern if k in hbm_bytes or k == "k_assign"), key=lambda k: kern[k]["total_ms"])
    if dom == "k_assign":
        ach = assign_flops / (kern[dom]["avg_us"] * 1e-6) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": counter_traffic(dom, sha, tag),
                "algorithmic_per_launch": assign_flops}
    else:
        per = hbm_bytes.get(dom)
        ach = per / (kern[dom]["avg_us"] * 1e-6) / 1e9 if per else None
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1) if ach else None, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4) if ach else None,
                "traffic": counter_traffic(dom, sha, tag), "algorithmic_per_launch": per}
    # every kernel's own roofline figure, for the record
    extra = {}
    for name, per in hbm_bytes.items():
        if name in kern:
            a = per / (kern[name]["avg_us"] * 1e-6) / 1e9
            extra[name] = {"bound": "hbm", "achieved_GBs": round(a, 1), "frac": round(a / HBM_PEAK_GBS, 4),
                           "bytes_per_launch": int(per), "traffic": counter_traffic(name, sha, tag)}
    if "k_assign" in kern:
        a = assign_flops / (kern["k_assign"]["avg_us"] * 1e-6) / 1e12
        extra["k_assign"] = {"bound": "mfma", "achieved_TFLOPs": round(a, 1), "frac": round(a / BF16_PEAK_TFLOPS, 4),
                             "flops_per_launch": assign_flops, "hbm_bytes_per_launch": int(assign_bytes),
                             "traffic": counter_traffic("k_assign", sha, tag)}

    decodes = args.steps * QPS
    build_ms = sum(kern[k]["total_ms"] for k in kern if k not in ("k_score", "k_topk", "k_attend", "k_merge"))
    build_tps = args.steps * int(ctx.sum()) / (build_ms / 1000.0)
    if QPS > 0:
        metric = ("sparse decode-attn steps/s (whole job: index build + %d decode queries per step), %s"
                  % (QPS, "8B-shape layer at 128K ctx" if headline else W["workload"]))
        value, unit = decodes / (t_plain / 1000.0), "decode steps/s"
    else:
        metric = "index-build tokens/s (segmented k-means + layout), %s" % W["workload"]
        value, unit = args.steps * int(ctx.sum()) / (t_plain / 1000.0), "tokens/s"
    cfg = dict(W)
    if isinstance(W["ctx"], list):
        cfg["ctx_per_sequence"] = [int(n) for n in ctx]
    result = {
        "metric": metric,
        "value": round(value, 1),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_plain / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": cfg,
        "roofline": roof,
        "decode_only_steps_per_s": round(decodes / (t_dec / 1000.0), 1) if QPS > 0 else None,
        "decode_only_us_per_query": round(1000.0 * t_dec / decodes, 2) if QPS > 0 else None,
        "decode_only_effective_GBs": round(step_bytes * decodes / (t_dec / 1000.0) / 1e9, 1) if QPS > 0 else None,
        "decode_bytes_per_query": int(step_bytes) if QPS > 0 else None,
        "build_tokens_per_s": round(build_tps, 1),
        "timing": "eager launches" if args.eager else "HIP graph replays",
        "eager_with_kernel_events_ms_per_step": round(t_ms / args.steps, 4),
        "kernels": {k: {"launches": v["launches"], "avg_us": round(v["avg_us"], 2)} for k, v in kern.items()},
        "kernel_roofline": extra,
        "source_sha": sha,
    }
    return result, (K, V, ctx, q)




def cpu_baseline(W, K, V, ctx, q, budget_s):
    """The oracle, as it stands, timed on this host's cores on a bounded sample of one step.

    One step = index build (every unit: B*G*ceil(N/seg) independent k-means problems, then
    the layout) + 64 decode queries. Sample: a few k-means units and a few decode queries
    against an oracle index over a prescribed clustering; the step time is extrapolated
    by the unit and query counts.
    """
    import numpy as np

    import oracle

    G, H, seg, K_s, iters = W["kv_heads"], W["q_heads"], W["seg_len"], W["clusters_per_seg"], W["kmeans_iters"]
    N = int(ctx[0])
    units_total = len(ctx) * G * (-(-N // seg))
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    t0 = time.time()
    n_units = 0
    while n_units < units_total and (n_units == 0 or time.time() - t0 < 0.5 * budget_s):
        key = oracle.seed_key(0, n_units // (N // seg), n_units % (N // seg))
        oracle.kmeans_segment(K[n_units * seg:(n_units + 1) * seg], K_s, iters, W["seed_build"], key=key)
        n_units += 1
    t_unit = (time.time() - t0) / n_units
    # decode sample on an oracle index over the generator's labels (k-means cost already sampled)
    lab = (np.arange(K.shape[0]) % seg) % K_s + (np.arange(K.shape[0]) % N) // seg * K_s
    t1 = time.time()
    idx = oracle.index_from_assign(K, V, G, ctx, seg, K_s, W["seed_build"], lab.astype(np.int32))
    t_layout = time.time() - t1
    n_tail = int(W.get("tail", 0))
    if n_tail:  # the decoded tokens of the GPU run
        import synth
        Kx, Vx, _ = synth.kv(W["seed_data"] + 1, len(ctx), G, np.array([n_tail] * len(ctx), np.int64), seg)
        Kx = Kx.reshape(len(ctx), G, n_tail, 128)
        Vx = Vx.reshape(len(ctx), G, n_tail, 128)
    t2 = time.time()
    n_dec = 0
    while n_dec < min(q.shape[0], W["decode_queries_per_step"]) and (n_dec == 0 or time.time() - t2 < 0.5 * budget_s):
        if n_tail:
            oracle.decode_tail(idx, K, V, q[n_dec], W["n_sink"], W["n_local"], W["topk_frac"], Kx, Vx,
                               [n_tail] * len(ctx))
        else:
            oracle.decode(idx, K, V, q[n_dec], W["n_sink"], W["n_local"], W["topk_frac"],
                          shared=W.get("shared", False))
        n_dec += 1
    t_dec = (time.time() - t2) / n_dec
    step_s = units_total * t_unit + t_layout + W["decode_queries_per_step"] * t_dec
    out = {"value": round(W["decode_queries_per_step"] / step_s, 4), "unit": "decode steps/s",
           "cores": threads, "kind": "oracle",
           "sample": "%d of %d k-means units (%.2f s each), one index layout (%.2f s), %d of 64 decode queries "
                     "(%.3f s each); step time %.1f s extrapolated" % (n_units, units_total, t_unit, t_layout, n_dec,
                                                                     t_dec, step_s)}
    out.update(cpu_info())
    # the same sample on one thread, in a child process (OpenMP reads its thread count at start)
    import subprocess
    try:
        env = dict(os.environ, OMP_NUM_THREADS="1")
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-single-thread"], env=env,
                           capture_output=True, text=True, timeout=120)
        one = json.loads(r.stdout.strip().splitlines()[-1])
        step1 = units_total * one["t_unit"] + one["t_layout"] + W["decode_queries_per_step"] * one["t_dec"]
        out["single_thread"] = {"value": round(W["decode_queries_per_step"] / step1, 5), "unit": "decode steps/s",
                                "cores": 1, "sample": "1 k-means unit (%.2f s), one index layout (%.2f s), 2 decode "
                                "queries (%.3f s each); step time %.1f s extrapolated"
                                % (one["t_unit"], one["t_layout"], one["t_dec"], step1)}
    except Exception as e:  # the figure is optional; the multi-thread baseline stands on its own
        out["single_thread"] = {"error": repr(e)[:200]}
    return out


def cpu_info():
    """CPU model, logical CPUs and the CPUs this process may run on."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "cpus_usable": len(os.sched_getaffinity(0))}


def cpu_single_thread_sample():
    """One k-means unit, one layout and two decode queries of the 128K layer's oracle on this process's
    threads (run with OMP_NUM_THREADS=1); prints their times as JSON."""
    import numpy as np

    import oracle
    import synth

    W = WORKLOAD
    G, seg, K_s, N = W["kv_heads"], W["seg_len"], W["clusters_per_seg"], W["ctx"]
    ctx = np.array([N], np.int64)
    K, V, _ = synth.kv(W["seed_data"], 1, G, ctx, seg)
    q, _ = synth.queries(W["seed_query"], 2, 1, W["q_heads"], G, ctx, K)
    t0 = time.time()
    oracle.kmeans_segment(K[:seg], K_s, W["kmeans_iters"], W["seed_build"], key=oracle.seed_key(0, 0, 0))
    t_unit = time.time() - t0
    lab = (np.arange(K.shape[0]) % seg) % K_s + (np.arange(K.shape[0]) % N) // seg * K_s
    t0 = time.time()
    idx = oracle.index_from_assign(K, V, G, ctx, seg, K_s, W["seed_build"], lab.astype(np.int32))
    t_layout = time.time() - t0
    t0 = time.time()
    for s in range(2):
        oracle.decode(idx, K, V, q[s], W["n_sink"], W["n_local"], W["topk_frac"])
    t_dec = (time.time() - t0) / 2
    print(json.dumps({"t_unit": t_unit, "t_layout": t_layout, "t_dec": t_dec}))





if __name__ == "__main__":
    main()
