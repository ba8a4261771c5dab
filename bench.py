"""Benchmark of the block-sparse prefill hot path on one MI355X.

One step = the whole path on one batch of synthetic input: block-mean
pooling + block scores + threshold + lists (fp_select_blocks), then attention
over the kept blocks with the mean correction (fp_sparse_prefill_fwd).  The
default workload is one Llama-3-8B-shaped layer at 131072 tokens (32 query
heads, 8 KV heads, d 128, block 128), threshold ratio 0.1; the ratios 0.05 and
0.2 are timed beside it.

Prints one JSON line.  value = effective TFLOP/s of the whole step, counting
only the algorithmic work of the executed blocks: F_kept = 4 d sum over kept
(h, I, J) of n_I n_J and F_corr = 4 d sum over (h, I) of n_I * |skipped J < I|.
The roofline entry is for the attention kernel (MFMA-bound), timed with HIP
events on the launch stream.  latency_spread gives the median and minimum of
the per-step selection, attention and step times; hbm_anchor the streaming
bandwidth of torch's own sum and copy kernels on the same GPU.  The CPU
baseline is the fp64 oracle on a bounded sample of the same workload.

Beside the headline: the fp8 layer, the paged batch (bf16 and fp8) and its
chunked variant (bf16 and fp8); the tiny (1K) and 32K workloads with their own latency,
effective TFLOP/s and alpha = 0 dense reference (`configs`); and, outside every
timed region, a parity summary of all five workloads against the oracle
(`parity`: mask mismatches inside and outside the threshold band, band size,
max-abs output error).
"""
import argparse
import json
import statistics
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse prefill attn latency + effective TFLOP/s (% MFMA peak) at 128K, GQA 32/8 d128"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBPS = 8000.0
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "k_attn_bf16_llama8b_s128k_traffic.json")
ATTN_SOURCES = ("k_attn.hip", "attn_walk.h", "fp_attn.h", "fp_device.h", "fp_launch.h")


def measured_traffic():
    """Calibrated HBM bytes per attention launch from the committed rocprofv3
    counter record, or None when the kernel sources changed since it was taken."""
    try:
        rec = json.load(open(TRAFFIC_RECORD))
    except (OSError, ValueError):
        return None
    if attn_source_hash() != rec.get("source_sha256"):
        return None
    return int(rec["traffic_bytes"])


def attn_source_hash():
    """sha256 of the attention kernel's sources with comments and blank lines
    left out, so that the traffic record stays valid across comment edits and
    reads null once the code changes."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        text = open(os.path.join(ROOT, "block_sparse_long_pooling_amd", "csrc", f)).read()
        for line in text.splitlines():
            code = re.sub(r"//.*$", "", line).rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()


def _short_name(name):
    """Kernel name without 'void', the anonymous namespace and the argument list."""
    name = name.replace("(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[5:]
    return name.split("(")[0]


def _counter_rows(folder):
    """(kernel name, counter, value) of every dispatch in the rocprofv3
    counter-collection CSV files under folder."""
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)):
        with open(f, newline="") as fh:
            for i, r in enumerate(csv.DictReader(fh)):
                did = r.get("Dispatch_Id") or r.get("Correlation_Id") or f"{f}:{i}"
                rows.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"]), did))
    return rows


def traffic_record(fetch_dir, write_dir):
    """Write the calibrated HBM-traffic record of the attention kernel from two
    rocprofv3 --pmc runs of `bench.py --quick --layouts --steps 2 --warmup 0
    --copy-probe` (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).  The 1 GiB
    device copy of --copy-probe calibrates each counter: factor = bytes the copy
    must move / bytes the counter reports for it.  Prints a per-kernel table."""
    per = {}
    for folder, counter in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        disp = {}
        for name, cname, val, did in _counter_rows(folder):
            if cname == counter:
                disp[(name, did)] = disp.get((name, did), 0.0) + val   # summed over the rows of a dispatch
        for (name, _), val in disp.items():
            per.setdefault(name, {}).setdefault(counter, []).append(val)
    # the probe's copy: a copy kernel with a dispatch that writes 1 GiB (within 1%)
    gib_kib = float(1 << 20)
    copy = [(n, i) for n in per if "copy" in n.lower() and "Cat" not in n
            for i, w in enumerate(per[n].get("WRITE_SIZE", [])) if abs(w / gib_kib - 1.0) < 0.01]
    if not copy:
        raise SystemExit("no 1 GiB copy dispatch found (run with --copy-probe)")
    cname, ci = copy[0]
    ff = gib_kib / per[cname]["FETCH_SIZE"][ci]
    wf = gib_kib / per[cname]["WRITE_SIZE"][ci]
    key = "k_attn_bf16<128, 128, 0>"          # the contiguous form
    attn = [n for n in per if key in n]
    if not attn:
        raise SystemExit(f"no {key} dispatch found")
    fk = statistics.mean(per[attn[0]]["FETCH_SIZE"])
    wk = statistics.mean(per[attn[0]]["WRITE_SIZE"])
    rec = {"kernel": key, "source_sha256": attn_source_hash(), "fetch_kib": fk, "write_kib": wk,
           "fetch_factor": ff, "write_factor": wf, "traffic_bytes": (fk * ff + wk * wf) * 1024.0,
           "commands": [
               f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o run -- "
               "python3 bench.py --quick --layouts --steps 2 --warmup 0 --copy-probe",
               f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o run -- "
               "python3 bench.py --quick --layouts --steps 2 --warmup 0 --copy-probe"]}
    with open(TRAFFIC_RECORD, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(f"copy calibration ({cname[:60]}): FETCH factor {ff:.4f}, WRITE factor {wf:.4f}")
    print("| kernel | dispatches | FETCH_SIZE (KiB, mean) | WRITE_SIZE (KiB, mean) | read (GiB) | write (GiB) |")
    print("|---|---|---|---|---|---|")
    for n in sorted(per):
        if not any(k in n for k in ("k_pool", "k_select", "k_quant", "k_attn")):
            continue
        f_ = statistics.mean(per[n].get("FETCH_SIZE", [0.0]))
        w_ = statistics.mean(per[n].get("WRITE_SIZE", [0.0]))
        print(f"| `{_short_name(n)}` | {len(per[n].get('FETCH_SIZE', []))} | {f_:.0f} | {w_:.0f} | "
              f"{f_ * ff / gib_kib:.3f} | {w_ * wf / gib_kib:.3f} |")
    print(f"record: {TRAFFIC_RECORD}: {rec['traffic_bytes']:.4g} bytes per attention launch")


def trace_summary(folder, timed):
    """Markdown table of this library's kernels from a rocprofv3 --kernel-trace
    --stats run: per kernel the launch count, the average over all launches
    (what --stats reports) and over the last `timed` launches (the timed
    steps), their min and max, then every kernel's durations in launch order
    (a kernel that several calls use lists their launches one call after the
    other)."""
    import csv
    import glob
    runs = {}
    for f in sorted(glob.glob(os.path.join(folder, "**", "*kernel_trace.csv"), recursive=True)):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"]
                if not any(k in name for k in ("k_pool", "k_select", "k_quant", "k_attn")):
                    continue
                us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                runs.setdefault(_short_name(name), []).append((int(r["Start_Timestamp"]), us))
    print(f"| kernel | launches | average, all (us) | average, last {timed} (us) | min (us) | max (us) |")
    print("|---|---|---|---|---|---|")
    for name in sorted(runs):
        d = [u for _, u in sorted(runs[name])]
        last = d[-timed:]
        print(f"| `{name}` | {len(d)} | {statistics.mean(d):.1f} | {statistics.mean(last):.1f} | "
              f"{min(last):.1f} | {max(last):.1f} |")
    print("\nLaunch durations in launch order (us):\n")
    for name in sorted(runs):
        print(f"- `{name}`: " + ", ".join(f"{u:.0f}" for _, u in sorted(runs[name])))


def counter_summary(folder):
    """Markdown table of this library's kernels from one rocprofv3 --pmc run:
    per kernel the mean of every counter per dispatch, and, when the counters
    are there, MFMA busy per SIMD (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE
    / 8 XCDs / 1024 SIMDs), vector instructions per MFMA, the LDS bank-conflict
    share and the share of wave cycles spent waiting."""
    per = {}
    for name, cname, val, disp in _counter_rows(folder):
        if not any(k in name for k in ("k_pool", "k_select", "k_quant", "k_attn")):
            continue
        per.setdefault(_short_name(name), {}).setdefault(cname, {}).setdefault(disp, 0.0)
        per[_short_name(name)][cname][disp] += val       # a counter may come per XCD / SE row
    counters = sorted({c for k in per.values() for c in k})
    derived = ["MFMA busy per SIMD", "VALU per MFMA", "LDS conflict share", "waiting share"]
    print("| kernel | dispatches | " + " | ".join(counters) + " | " + " | ".join(derived) + " |")
    print("|---|---|" + "---|" * (len(counters) + len(derived)))
    for name in sorted(per):
        mean = {c: statistics.mean(per[name][c].values()) for c in per[name]}
        nd = max(len(per[name][c]) for c in per[name])
        g = lambda c: mean.get(c)
        d = []
        d.append(f"{100 * g('SQ_VALU_MFMA_BUSY_CYCLES') / (g('GRBM_GUI_ACTIVE') / 8) / 1024:.1f}%"
                 if g("SQ_VALU_MFMA_BUSY_CYCLES") is not None and g("GRBM_GUI_ACTIVE") else "-")
        d.append(f"{g('SQ_INSTS_VALU') / g('SQ_INSTS_MFMA'):.2f}" if g("SQ_INSTS_MFMA") else "-")
        d.append(f"{100 * g('SQ_LDS_BANK_CONFLICT') / g('SQ_LDS_IDX_ACTIVE'):.1f}%"
                 if g("SQ_LDS_IDX_ACTIVE") and g("SQ_LDS_BANK_CONFLICT") is not None else "-")
        d.append(f"{100 * g('SQ_WAIT_INST_ANY') / g('SQ_WAVE_CYCLES'):.0f}%"
                 if g("SQ_WAVE_CYCLES") and g("SQ_WAIT_INST_ANY") is not None else "-")
        print(f"| `{name}` | {nd} | " + " | ".join(f"{mean[c]:.4e}" if c in mean else "-" for c in counters)
              + " | " + " | ".join(d) + " |")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b_s128k")
    ap.add_argument("--alpha", type=float, default=0.1)
    ap.add_argument("--no-correction", action="store_true")
    ap.add_argument("--quick", action="store_true",
                    help="headline alpha only: no sweep, no dense references, no CPU baseline")
    ap.add_argument("--layouts", action="store_true",
                    help="with --quick: still time the fp8 layer and the paged batch")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--configs", action="store_true",
                    help="with --quick: still time the tiny (1K) and 32K workloads")
    ap.add_argument("--parity", action="store_true", help="with --quick: still run the parity summary")
    ap.add_argument("--no-parity", action="store_true", help="skip the parity summary")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 1 GiB device copy (calibrates the HBM byte counters)")
    ap.add_argument("--traffic-record", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: write the attention kernel's calibrated traffic record from two "
                         "rocprofv3 --pmc output folders (FETCH_SIZE, WRITE_SIZE) and print a table")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR",
                    help="no GPU work: print a table of this library's kernels from a rocprofv3 --kernel-trace "
                         "run (averages over all launches and over the last --steps launches)")
    ap.add_argument("--counter-summary", metavar="PMC_DIR",
                    help="no GPU work: print a table of this library's kernels from one rocprofv3 --pmc run")
    return ap.parse_args()


def work_counts(fp, sel, S, Hq, d, B, correction):
    """F_kept, F_corr and kept-block count from the device lists."""
    import torch
    nB = (S + B - 1) // B
    cnt = sel.kv_cnt.to(torch.int64)                                    # [Hq, nB]
    I = torch.arange(nB, device=cnt.device)
    base = (torch.arange(Hq, device=cnt.device)[:, None] * (nB * (nB + 1) // 2)
            + (I * (I + 1) // 2)[None, :])
    last = sel.kv_idx.to(torch.int64)[base + cnt - 1]                  # largest kept J per row
    diag_kept = (last == I[None, :]).to(torch.int64)
    n = torch.full((nB,), B, dtype=torch.int64, device=cnt.device)
    n[-1] = S - (nB - 1) * B
    # only row nB-1 can hold the partial block, and only as its diagonal
    n_j_sum = cnt * B
    n_j_sum[:, -1] -= diag_kept[:, -1] * (B - int(n[-1]))
    f_kept = 4.0 * d * float((n[None, :] * n_j_sum).sum())
    f_corr = 0.0
    if correction:
        skipped = I[None, :] - (cnt - diag_kept)
        f_corr = 4.0 * d * float((n[None, :] * skipped).sum())
    return f_kept, f_corr, int(cnt.sum())


def selection_bytes(S, Hq, Hkv, d, B, kept, correction):
    nB = (S + B - 1) // B
    nv = 1 if correction else 0
    read = S * (Hq + Hkv * (1 + nv)) * d * 2
    write = (Hq + Hkv * (1 + nv)) * nB * d * 4 + 4 * kept + 4 * Hq * nB
    return read + write


def time_steps(fn_sel, fn_attn, steps, stream):
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record(stream)
        fn_sel()
        e1.record(stream)
        fn_attn()
        e2.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sel = [a.elapsed_time(b) for a, b, _ in ev]
    attn = [b.elapsed_time(c) for _, b, c in ev]
    total = [a.elapsed_time(c) for a, _, c in ev]
    spread = {name: {"median": round(statistics.median(x), 4), "min": round(min(x), 4)}
              for name, x in (("select_ms", sel), ("attn_ms", attn), ("step_ms", total))}
    return wall * 1e3 / steps, sum(sel) / steps, sum(attn) / steps, spread


def main():
    args = parse()
    if args.traffic_record:
        traffic_record(*args.traffic_record)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary, args.steps)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): the path is built and "
              "timed on a single MI355X; see the design notes for how it would shard.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import block_sparse_long_pooling_amd as fp
    from block_sparse_long_pooling_amd import synth

    w = synth.WORKLOADS[args.workload]
    if w.paged or w.dtype != "bf16":
        raise SystemExit("bench.py times the single-sequence bf16 workloads")
    S, Hq, Hkv, d, B = w.seqlens[0], w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    corr = not args.no_correction
    log(f"bench: workload {w.name} S={S} Hq={Hq} Hkv={Hkv} d={d} B={B} alpha={args.alpha} corr={corr}")
    t = time.perf_counter()
    q, k, v = synth.make_sequence(S, Hq, Hkv, d, w.seed, w.verticals)
    log(f"bench: inputs generated in {time.perf_counter() - t:.1f}s")
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    stream = torch.cuda.current_stream(dev)
    out = torch.empty((S, Hq, d), dtype=torch.bfloat16, device=dev)
    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def measure(alpha, steps, warmup, shared=False, probes=0):
        p = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=corr, shared_selection=shared,
                           query_probes=probes)
        sel = fp.alloc_selection(p, S, dev)
        fs = lambda: fp.fp_select_blocks(p, qd, kd, vd, sel=sel)
        fa = lambda: fp.fp_sparse_prefill_fwd(p, qd, kd, vd, sel, out=out)
        for _ in range(warmup):
            fs(); fa()
        step_ms, sel_ms, attn_ms, spread = time_steps(fs, fa, steps, stream)
        f_kept, f_corr, kept = work_counts(fp, sel, S, Hq, d, B, corr)
        causal = Hq * ((S + B - 1) // B) * ((S + B - 1) // B + 1) // 2
        return dict(alpha=alpha, ms_per_step=step_ms, select_ms=sel_ms, attn_ms=attn_ms, spread=spread,
                    f_kept=f_kept, f_corr=f_corr, kept_blocks=kept, density=kept / causal,
                    sel=sel, p=p)

    head = measure(args.alpha, args.steps, args.warmup)
    f_alg = head["f_kept"] + head["f_corr"]
    attn_tflops = f_alg / (head["attn_ms"] * 1e-3) / 1e12
    step_tflops = f_alg / (head["ms_per_step"] * 1e-3) / 1e12
    sel_bytes = selection_bytes(S, Hq, Hkv, d, B, head["kept_blocks"], corr)
    sel_gbps = sel_bytes / (head["select_ms"] * 1e-3) / 1e9
    log(f"bench: alpha={args.alpha} step {head['ms_per_step']:.3f} ms (select {head['select_ms']:.3f}, "
        f"attn {head['attn_ms']:.3f}); density {head['density']:.4f}; attn {attn_tflops:.1f} TFLOP/s; "
        f"select {sel_gbps:.0f} GB/s")

    extra = {"latency_spread": head["spread"]}
    if not args.quick:
        extra["hbm_anchor"] = hbm_anchor(stream, dev)
        log(f"bench: hbm anchor {extra['hbm_anchor']}")
        sweep = []
        for a in w.alphas:
            if a == args.alpha:
                continue
            r = measure(a, max(3, args.steps // 2), 1)
            fa_ = r["f_kept"] + r["f_corr"]
            sweep.append(dict(alpha=a, ms_per_step=round(r["ms_per_step"], 4),
                              select_ms=round(r["select_ms"], 4), attn_ms=round(r["attn_ms"], 4),
                              density=round(r["density"], 5),
                              attn_tflops=round(fa_ / (r["attn_ms"] * 1e-3) / 1e12, 2)))
            log(f"bench: sweep {sweep[-1]}")
            del r
        extra["alpha_sweep"] = sweep
        # group-shared selection: one list per KV head, the union of its query
        # heads' lists, or the list of the group-pooled query
        for mode, key in (("union", "shared_selection"), ("pooled", "shared_selection_pooled")):
            r = measure(args.alpha, max(3, args.steps // 2), 1, shared=mode)
            fa_ = r["f_kept"] + r["f_corr"]
            jac = mask_agreement(head["sel"], r["sel"], S, Hq, B, dev)
            extra[key] = dict(alpha=args.alpha, ms_per_step=round(r["ms_per_step"], 4),
                              select_ms=round(r["select_ms"], 4), attn_ms=round(r["attn_ms"], 4),
                              density=round(r["density"], 5),
                              attn_tflops=round(fa_ / (r["attn_ms"] * 1e-3) / 1e12, 2),
                              kept_jaccard_vs_per_head=round(jac, 4))
            log(f"bench: {key} {extra[key]}")
            del r
        # skeleton-query scoring: q_bar from 16 uniformly spaced queries per block
        r = measure(args.alpha, max(3, args.steps // 2), 1, probes=16)
        fa_ = r["f_kept"] + r["f_corr"]
        jac = mask_agreement(head["sel"], r["sel"], S, Hq, B, dev)
        extra["skeleton_queries"] = dict(alpha=args.alpha, probes=16, ms_per_step=round(r["ms_per_step"], 4),
                                         select_ms=round(r["select_ms"], 4), attn_ms=round(r["attn_ms"], 4),
                                         density=round(r["density"], 5),
                                         attn_tflops=round(fa_ / (r["attn_ms"] * 1e-3) / 1e12, 2),
                                         kept_jaccard_vs_full_pooling=round(jac, 4))
        log(f"bench: skeleton queries {extra['skeleton_queries']}")
        del r
        # dense references on the same GPU
        dense = measure(0.0, 2, 1)
        f_dense = 4.0 * d * Hq * (S * (S + 1) / 2)
        extra["dense_ref"] = {
            "ours_alpha0_attn_ms": round(dense["attn_ms"], 3),
            "ours_alpha0_tflops": round(f_dense / (dense["attn_ms"] * 1e-3) / 1e12, 1),
        }
        del dense
        torch.cuda.empty_cache()
        try:
            Qt = qd.permute(1, 0, 2)[None]
            Kt = kd.permute(1, 0, 2)[None]
            Vt = vd.permute(1, 0, 2)[None]
            f = lambda: torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt, is_causal=True,
                                                                         enable_gqa=True)
            f()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(2):
                f()
            e1.record(stream)
            torch.cuda.synchronize()
            sdpa_ms = e0.elapsed_time(e1) / 2
            extra["dense_ref"]["torch_sdpa_ms"] = round(sdpa_ms, 3)
            extra["dense_ref"]["torch_sdpa_tflops"] = round(f_dense / (sdpa_ms * 1e-3) / 1e12, 1)
            extra["dense_ref"]["speedup_vs_torch_sdpa"] = round(sdpa_ms / head["ms_per_step"], 2)
        except Exception as ex:          # black-box reference; report, do not fail the bench
            extra["dense_ref"]["torch_sdpa_error"] = str(ex)[:200]
        log(f"bench: dense {extra['dense_ref']}")

    if not args.quick or args.layouts:
        extra.update(other_layouts(fp, synth, q, k, v, head, stream, dev, corr))

    if not args.quick or args.configs:
        extra["configs"] = [small_config(fp, synth, name, corr, args.steps, args.warmup, stream, dev)
                            for name in ("tiny_s1k_gqa4_d64", "llama8b_s32k")]

    cpu = None
    oracle128 = []
    if not args.quick:
        cpu = cpu_baseline(q, k, v, B, args.alpha, corr, head, args.cpu_seconds, oracle128)
        log(f"bench: cpu {cpu}")
    if (not args.quick and not args.no_parity) or args.parity:
        del head["sel"]
        torch.cuda.empty_cache()
        extra["parity"] = parity_summary(fp, synth, dev, corr, q, k, v, oracle128[0] if oracle128 else None)

    roof = {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "kernel": "k_attn_bf16<128,128>", "traffic": measured_traffic(),
            "traffic_unit": "bytes/launch (FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0, copy-calibrated)"}
    rec = {
        "metric": METRIC, "value": round(step_tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "seq_len": S, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "block": B, "alpha": args.alpha, "mean_correction": corr},
        "select_ms": round(head["select_ms"], 4), "attn_ms": round(head["attn_ms"], 4),
        "density": round(head["density"], 5), "attn_tflops": round(attn_tflops, 2),
        "select_gbps": round(sel_gbps, 1), "select_hbm_frac": round(sel_gbps / PEAK_HBM_GBPS, 4),
        "flops": {"kept": head["f_kept"], "corr": head["f_corr"]},
        # beside the headline: the kept blocks' share alone, and the dense
        # causal work (4 d Hq S^2 / 2) over the sparse attention time -- a
        # dense-equivalent rate, not work the kernel does
        "attn_kept_tflops": round(head["f_kept"] / (head["attn_ms"] * 1e-3) / 1e12, 2),
        "attn_dense_equivalent_tflops": round(4.0 * d * Hq * S * S / 2 / (head["attn_ms"] * 1e-3) / 1e12, 1),
        "roofline": roof, "cpu_baseline": cpu,
    }
    rec.update(extra)
    print(json.dumps(rec), flush=True)


def mask_agreement(sel_a, sel_b, S, Hq, B, dev):
    """|A and B| / |A or B| over the kept (head, query block, KV block) triples
    of two single-sequence selections."""
    import torch
    nB = (S + B - 1) // B

    def mask(sel):
        cnt = sel.kv_cnt.reshape(-1).to(torch.int64)                          # [Hq * nB], row = h * nB + I
        rows = torch.arange(Hq * nB, device=dev)
        h, I = rows // nB, rows % nB
        base = h * (nB * (nB + 1) // 2) + I * (I + 1) // 2
        r = torch.repeat_interleave(rows, cnt)
        j = torch.arange(int(cnt.sum()), device=dev) - torch.repeat_interleave(torch.cumsum(cnt, 0) - cnt, cnt)
        cols = sel.kv_idx.to(torch.int64)[torch.repeat_interleave(base, cnt) + j]
        m = torch.zeros(Hq * nB * nB, dtype=torch.bool, device=dev)
        m[r * nB + cols] = True
        return m

    a, b = mask(sel_a), mask(sel_b)
    return float((a & b).sum()) / max(1.0, float((a | b).sum()))


def hbm_anchor(stream, dev):
    """Streaming bandwidth of torch's own kernels on this GPU, as a sanity
    anchor for the 8 TB/s peak: a 4 GiB fp32 sum (read), a 2 GiB copy (read +
    write), and a bf16 -> e4m3 conversion of 1.5 GiB (2 bytes read per byte
    written: the read/write mix of the fused fp8 preparation)."""
    import torch
    buf = torch.ones(1 << 30, dtype=torch.float32, device=dev)
    t_sum = timed_ms(lambda: buf.sum(), 5, stream)
    src = buf[: 1 << 29]
    dst = torch.empty_like(src)
    t_copy = timed_ms(lambda: dst.copy_(src), 5, stream)
    del buf, src, dst
    src16 = torch.ones(3 << 28, dtype=torch.bfloat16, device=dev)
    dst8 = torch.empty(3 << 28, dtype=torch.float8_e4m3fn, device=dev)
    t_cvt = timed_ms(lambda: dst8.copy_(src16), 5, stream)
    del src16, dst8
    return {"torch_sum_read_gbps": round(4 * (1 << 30) / (t_sum * 1e-3) / 1e9, 1),
            "torch_copy_gbps": round(2 * 4 * (1 << 29) / (t_copy * 1e-3) / 1e9, 1),
            "torch_bf16_to_fp8_gbps": round(3 * (3 << 28) / (t_cvt * 1e-3) / 1e9, 1)}


def timed_ms(fn, n, stream):
    import torch
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def other_layouts(fp, synth, q, k, v, head, stream, dev, corr):
    """The other input layouts of the path, timed beside the headline: the
    same 128K layer in fp8 e4m3 (one fused pass writes the codes, the
    per-(head, block) scales, the block means and the lists; selection is on
    the bf16 data, so the lists are the headline's up to threshold-band
    rounding; then fp8 attention), the paged continuous batch of 8 requests
    (selection and attention in one call), and the same batch as chunked
    prefill, in bf16 and with fp8 attention."""
    import torch
    res = {}
    S, Hq, d = q.shape
    Hkv = k.shape[1]
    B = head["p"].block_size
    # fp8: one pass over the bf16 Q/K/V writes e4m3 codes, scales, block means
    # and the lists; attention then reads the codes.
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    p8 = fp.make_params(Hq, Hkv, d, B, head["alpha"], mean_correction=corr, dtype=fp.FP_DTYPE_FP8_E4M3FN)
    sel8, f8 = fp.fp_select_blocks_fp8(p8, qd, kd, vd)
    tp = timed_ms(lambda: fp.fp_select_blocks_fp8(p8, qd, kd, vd, sel=sel8, f8=f8), 5, stream)
    out = torch.empty((S, Hq, d), dtype=torch.bfloat16, device=dev)
    t8 = timed_ms(lambda: fp.fp_sparse_prefill_fwd(p8, f8.q8, f8.k8, f8.v8, sel8, q_scale=f8.q_scale,
                                                   k_scale=f8.k_scale, v_scale=f8.v_scale, out=out), 5, stream)
    f_kept, f_corr, kept = work_counts(fp, sel8, S, Hq, d, B, corr)
    f_alg = f_kept + f_corr
    nB = (S + B - 1) // B
    ntok = S * (Hq + 2 * Hkv) * d
    prep_bytes = (3 * ntok + 4 * (Hq + 2 * Hkv) * nB + 4 * (Hq + Hkv) * nB * d
                  + (4 * Hkv * nB * d if corr else 0) + 4 * kept + 4 * Hq * nB)
    res["fp8"] = {"workload": "llama8b_s128k_fp8", "dtype": "fp8_e4m3",
                  "prep_ms": round(tp, 4), "prep_gbps": round(prep_bytes / (tp * 1e-3) / 1e9, 1),
                  "attn_ms": round(t8, 4), "step_ms": round(tp + t8, 4),
                  "attn_tflops": round(f_alg / (t8 * 1e-3) / 1e12, 2),
                  "frac_fp8_peak": round(f_alg / (t8 * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)}
    log(f"bench: fp8 {res['fp8']}")
    del qd, kd, vd, out, sel8, f8
    torch.cuda.empty_cache()

    w = synth.WORKLOADS["paged_batch8"]
    pb = synth.workload_inputs(w, keep_requests=False)
    p = fp.make_params(w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, head["alpha"],
                       mean_correction=corr)
    qd, kc, vc, bt = (x.to(dev) for x in (pb.q, pb.k_cache, pb.v_cache, pb.block_table))
    r = fp.fp_sparse_prefill_varlen_paged(p, qd, kc, vc, bt, pb.cu_seqlens)
    tv = timed_ms(lambda: fp.fp_sparse_prefill_varlen_paged(p, qd, kc, vc, bt, pb.cu_seqlens,
                                                            workspace=r.workspace, out=r.out), 5, stream)
    cu = [int(x) for x in pb.cu_seqlens]
    lens = [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]
    Bp, dp, Hqp = w.block_size, w.head_dim, w.num_q_heads
    kept, skipped = list_work(r.kv_idx, r.kv_cnt, lens, [0] * len(lens), Hqp, Bp, dev)
    # every request length is a multiple of the block, so all blocks are full:
    # a kept block costs B keys per query row, a skipped past block one pooled entry
    f_v = 4.0 * dp * Bp * (Bp * kept + (skipped if corr else 0))
    res["paged"] = {"workload": w.name, "tokens": cu[-1], "requests": len(cu) - 1, "step_ms": round(tv, 4),
                    "tokens_per_s": round(cu[-1] / (tv * 1e-3), 1), "kept_blocks": kept,
                    "tflops": round(f_v / (tv * 1e-3) / 1e12, 2)}
    log(f"bench: paged {res['paged']}")

    # The same batch in fp8: one pass writes the e4m3 paged cache, the Q codes
    # and the means; selection on the bf16 means; fp8 attention on the pages.
    p8 = fp.make_params(w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, head["alpha"],
                        mean_correction=corr, dtype=fp.FP_DTYPE_FP8_E4M3FN)
    r8, c8 = fp.fp_sparse_prefill_varlen_paged_fp8(p8, qd, kc, vc, bt, pb.cu_seqlens)
    t8 = timed_ms(lambda: fp.fp_sparse_prefill_varlen_paged_fp8(p8, qd, kc, vc, bt, pb.cu_seqlens, cache=c8,
                                                                workspace=r8.workspace, out=r8.out), 5, stream)
    kept8, skipped8 = list_work(r8.kv_idx, r8.kv_cnt, lens, [0] * len(lens), Hqp, Bp, dev)
    f_8 = 4.0 * dp * Bp * (Bp * kept8 + (skipped8 if corr else 0))
    res["paged_fp8"] = {"workload": w.name + "_fp8", "dtype": "fp8_e4m3", "tokens": cu[-1],
                        "step_ms": round(t8, 4), "tokens_per_s": round(cu[-1] / (t8 * 1e-3), 1),
                        "kept_blocks": kept8, "tflops": round(f_8 / (t8 * 1e-3) / 1e12, 2)}
    log(f"bench: paged fp8 {res['paged_fp8']}")
    del r8

    # Chunked prefill on the same contexts: the last CHUNK tokens of each
    # request are new; the prefix means were pooled into the cache by an
    # earlier call (untimed), the timed call reads them from it.
    CHUNK = 4096
    cut = [max(0, L - CHUNK) for L in lens]
    num_pages = kc.shape[0]
    cache = fp.alloc_pooled_cache(p, num_pages, dev)
    q_pre = torch.cat([qd[cu[b]:cu[b] + cut[b]] for b in range(len(lens))])
    cu_pre = [0]
    for c_ in cut:
        cu_pre.append(cu_pre[-1] + c_)
    fp.fp_sparse_prefill_chunked_paged(p, q_pre, kc, vc, bt, cu_pre, cut, pooled_cache=cache)
    q_new = torch.cat([qd[cu[b] + cut[b]:cu[b + 1]] for b in range(len(lens))])
    cu_new = [0]
    for b in range(len(lens)):
        cu_new.append(cu_new[-1] + lens[b] - cut[b])
    rc = fp.fp_sparse_prefill_chunked_paged(p, q_new, kc, vc, bt, cu_new, lens, pooled_cache=cache,
                                            prefix_pooled=True)
    tc = timed_ms(lambda: fp.fp_sparse_prefill_chunked_paged(p, q_new, kc, vc, bt, cu_new, lens,
                                                             pooled_cache=cache, prefix_pooled=True,
                                                             workspace=rc.workspace, out=rc.out), 5, stream)
    kept, skipped = list_work(rc.kv_idx, rc.kv_cnt, lens, cut, Hqp, Bp, dev)
    f_c = 4.0 * dp * Bp * (Bp * kept + (skipped if corr else 0))
    res["chunked"] = {"workload": w.name + "_last4096", "new_tokens": cu_new[-1],
                      "context_tokens": cu[-1], "chunk": CHUNK, "step_ms": round(tc, 4),
                      "new_tokens_per_s": round(cu_new[-1] / (tc * 1e-3), 1), "kept_blocks": kept,
                      "tflops": round(f_c / (tc * 1e-3) / 1e12, 2)}
    log(f"bench: chunked {res['chunked']}")

    # The same chunks with fp8 attention: the e4m3 pages of the prefixes are
    # those the fp8 paged call wrote; the timed call encodes the chunks' query
    # blocks (Q into its workspace, K and V into the pages) and reads the
    # prefix means from the same pooled cache.
    r8c = fp.fp_sparse_prefill_chunked_paged_fp8(p8, q_new, kc, vc, bt, cu_new, lens, c8, pooled_cache=cache,
                                                 prefix_pooled=True)
    tc8 = timed_ms(lambda: fp.fp_sparse_prefill_chunked_paged_fp8(p8, q_new, kc, vc, bt, cu_new, lens, c8,
                                                                  pooled_cache=cache, prefix_pooled=True,
                                                                  workspace=r8c.workspace, out=r8c.out),
                   5, stream)
    kept8, skipped8 = list_work(r8c.kv_idx, r8c.kv_cnt, lens, cut, Hqp, Bp, dev)
    f_c8 = 4.0 * dp * Bp * (Bp * kept8 + (skipped8 if corr else 0))
    res["chunked_fp8"] = {"workload": w.name + "_last4096_fp8", "dtype": "fp8_e4m3", "new_tokens": cu_new[-1],
                          "context_tokens": cu[-1], "chunk": CHUNK, "step_ms": round(tc8, 4),
                          "new_tokens_per_s": round(cu_new[-1] / (tc8 * 1e-3), 1), "kept_blocks": kept8,
                          "tflops": round(f_c8 / (tc8 * 1e-3) / 1e12, 2)}
    log(f"bench: chunked fp8 {res['chunked_fp8']}")
    del r8c, c8
    return res


def list_work(kv_idx, kv_cnt, kv_lens, starts, Hq, B, dev):
    """(kept, skipped past) block counts over all (head, query block) rows of
    lists in the paged/chunked layout: per request, rows of query blocks
    first .. nb-1 (first = start / B), row I with capacity I + 1."""
    import torch
    idx = kv_idx.to(torch.int64)
    cnt = kv_cnt.to(torch.int64)
    tri = lambda n: n * (n + 1) // 2
    kept = skipped = 0
    io = co = 0
    for L, P0 in zip(kv_lens, starts):
        nb, first = (L + B - 1) // B, P0 // B
        nq = nb - first
        if nq <= 0:
            continue
        c = cnt[co:co + Hq * nq].view(Hq, nq)
        I = torch.arange(first, nb, device=dev)
        rows = (io + torch.arange(Hq, device=dev)[:, None] * (tri(nb) - tri(first))
                + (I * (I + 1) // 2 - tri(first))[None, :])
        diag = (idx[rows + c - 1] == I[None, :]).to(torch.int64)
        kept += int(c.sum())
        skipped += int((I[None, :] - (c - diag)).sum())
        io += Hq * (tri(nb) - tri(first))
        co += Hq * nq
    return kept, skipped


def small_config(fp, synth, name, corr, steps, warmup, stream, dev):
    """One single-sequence workload at its threshold ratio: selection,
    attention and step latency, effective TFLOP/s (F_kept + F_corr over the
    attention and step times), density; our alpha = 0 kernel (every causal
    block) as the dense reference on the same GPU."""
    import torch
    w = synth.WORKLOADS[name]
    S, Hq, Hkv, d, B = w.seqlens[0], w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    q, k, v = synth.make_sequence(S, Hq, Hkv, d, w.seed, w.verticals)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty((S, Hq, d), dtype=torch.bfloat16, device=dev)
    nB = (S + B - 1) // B
    res = {"workload": name, "seq_len": S, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d, "block": B}
    for alpha in (w.alphas[0], 0.0):
        p = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=corr)
        sel = fp.alloc_selection(p, S, dev)
        fs = lambda: fp.fp_select_blocks(p, qd, kd, vd, sel=sel)
        fa = lambda: fp.fp_sparse_prefill_fwd(p, qd, kd, vd, sel, out=out)
        for _ in range(warmup):
            fs()
            fa()
        step_ms, sel_ms, attn_ms, spread = time_steps(fs, fa, steps if alpha > 0 else max(3, steps // 4), stream)
        f_kept, f_corr, kept = work_counts(fp, sel, S, Hq, d, B, corr)
        f = f_kept + f_corr
        if alpha > 0:
            res.update({"alpha": alpha, "select_ms": round(sel_ms, 4), "attn_ms": round(attn_ms, 4),
                        "step_ms": round(step_ms, 4), "latency_spread": spread,
                        "density": round(kept / (Hq * nB * (nB + 1) // 2), 5),
                        "attn_tflops": round(f / (attn_ms * 1e-3) / 1e12, 2),
                        "step_tflops": round(f / (step_ms * 1e-3) / 1e12, 2),
                        "attn_frac_bf16_peak": round(f / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                        "flops": {"kept": f_kept, "corr": f_corr}})
        else:
            res["dense_ref"] = {"ours_alpha0_attn_ms": round(attn_ms, 4),
                                "ours_alpha0_tflops": round(f / (attn_ms * 1e-3) / 1e12, 2),
                                "speedup_step_vs_alpha0_attn": round(attn_ms / res["step_ms"], 2)}
    log(f"bench: {name} {res}")
    return res


def _mask_stats(mask, ref_keep, ref_band):
    diff = mask != ref_keep
    return {"kept": int(mask.sum()), "band": int(ref_band.sum()),
            "mismatch_in_band": int((diff & ref_band).sum()),
            "mismatch_outside_band": int((diff & ~ref_band).sum())}


def _sampled_error(O, q, k, v, sel, keep, corr, out, pairs, B):
    """max |o_gpu - o_oracle| over the rows of the sampled (head, query block)
    pairs, the oracle run under the GPU's mask."""
    import numpy as np
    o_ref, _ = O.sparse_attention(q, k, v, sel, corr, pairs=pairs, keep=keep)
    err = 0.0
    S = q.shape[0]
    for h, I in pairs:
        r0, r1 = I * B, min(S, (I + 1) * B)
        err = max(err, float(np.abs(out[r0:r1, h] - o_ref[r0:r1, h]).max()))
    return err


def parity_summary(fp, synth, dev, corr, q128, k128, v128, oracle128=None):
    """Parity of every configuration against the CPU oracle, outside the timed
    regions: mask mismatches inside and outside the 1e-3 band around each
    threshold (outside must be 0), band size, and the max-abs output error
    against the oracle under the GPU's mask (whole output for the tiny
    workload, sampled (head, query block) pairs for the others; fp8 against
    the oracle on the oracle's own dequantized codes)."""
    import numpy as np
    import torch
    import oracle as O
    rng = np.random.default_rng(7)
    res = {}

    def single(name, alphas, q, k, v, full_error, npairs, sel_ref=None):
        S, Hq, d = q.shape
        Hkv = k.shape[1]
        B = synth.WORKLOADS[name].block_size
        nB = (S + B - 1) // B
        qn, kn, vn = q.float().numpy(), k.float().numpy(), v.float().numpy()
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        ref = sel_ref if sel_ref is not None else O.select_blocks(qn, kn, vn, B, alphas[0])
        out_cfg = {}
        for alpha in alphas:
            p = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=corr)
            sel = fp.fp_select_blocks(p, qd, kd, vd)
            mask = fp.lists_to_mask(sel.kv_idx, sel.kv_cnt, Hq, nB)
            keep, band = O.threshold(ref.score, alpha)
            st = _mask_stats(mask, keep, band)
            if alpha == alphas[0]:
                o = fp.fp_sparse_prefill_fwd(p, qd, kd, vd, sel).float().cpu().numpy()
                if full_error:
                    o_ref, _ = O.sparse_attention(qn, kn, vn, ref, corr, keep=mask)
                    st["max_abs_err"] = float(np.abs(o - o_ref).max())
                    st["err_rows"] = "all"
                else:
                    pairs = [divmod(int(x), nB) for x in rng.choice(Hq * nB, npairs, replace=False)]
                    st["max_abs_err"] = _sampled_error(O, qn, kn, vn, ref, mask, corr, o, pairs, B)
                    st["err_rows"] = f"{npairs} random (head, query block) pairs"
            out_cfg[str(alpha)] = st
        return out_cfg, ref

    t0 = time.perf_counter()
    w = synth.WORKLOADS["tiny_s1k_gqa4_d64"]
    q, k, v = synth.make_sequence(w.seqlens[0], w.num_q_heads, w.num_kv_heads, w.head_dim, w.seed, w.verticals)
    res[w.name], _ = single(w.name, (0.1, 0.3, 0.5, 0.9), q, k, v, True, 0)
    w = synth.WORKLOADS["llama8b_s32k"]
    q, k, v = synth.make_sequence(w.seqlens[0], w.num_q_heads, w.num_kv_heads, w.head_dim, w.seed, w.verticals)
    res[w.name], _ = single(w.name, (0.1,), q, k, v, False, 16)
    del q, k, v
    res["llama8b_s128k"], ref128 = single("llama8b_s128k", (0.1, 0.05, 0.2), q128, k128, v128, False, 16,
                                          oracle128)
    # fp8: lists from the fused fp8 preparation (selection on the bf16 data),
    # output against the oracle on the oracle's own codes of KV head 0's group
    Hq, Hkv = q128.shape[1], k128.shape[1]
    g = Hq // Hkv
    S, d = q128.shape[0], q128.shape[2]
    B = 128
    nB = S // B
    p8 = fp.make_params(Hq, Hkv, d, B, 0.1, mean_correction=corr, dtype=fp.FP_DTYPE_FP8_E4M3FN)
    sel8, f8 = fp.fp_select_blocks_fp8(p8, q128.to(dev), k128.to(dev), v128.to(dev))
    o8 = fp.fp_sparse_prefill_fwd(p8, f8.q8, f8.k8, f8.v8, sel8, q_scale=f8.q_scale, k_scale=f8.k_scale,
                                  v_scale=f8.v_scale).float().cpu().numpy()
    mask8 = fp.lists_to_mask(sel8.kv_idx, sel8.kv_cnt, Hq, nB)
    keep, band = O.threshold(ref128.score, 0.1)
    st = _mask_stats(mask8, keep, band)
    del sel8, f8
    deq = []
    for x in (q128[:, :g], k128[:, :1], v128[:, :1]):
        c, sc = O.quantize_fp8_blockwise(x.float().numpy(), B)
        deq.append(O.dequantize_blockwise(synth.fp8_codes_to_float(torch.from_numpy(c)).numpy(), sc, B))
    sub = O.Selection(None, ref128.k_bar[:1], ref128.v_bar[:1], None, None, None, None, B)
    pairs = [(int(h), int(I)) for h, I in zip(rng.integers(0, g, 12), rng.integers(0, nB, 12))]
    st["max_abs_err"] = _sampled_error(O, deq[0], deq[1], deq[2], sub, mask8[:g], corr, o8[:, :g], pairs, B)
    st["err_rows"] = "12 random (head, query block) pairs of KV head 0's query heads, oracle on its own e4m3 codes"
    res["llama8b_s128k_fp8"] = {"0.1": st}
    del deq, o8
    # paged batch: each request against the oracle run on it alone
    w = synth.WORKLOADS["paged_batch8"]
    pb = synth.workload_inputs(w, keep_requests=True)
    p = fp.make_params(w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, 0.1, mean_correction=corr)
    r = fp.fp_sparse_prefill_varlen_paged(p, pb.q.to(dev), pb.k_cache.to(dev), pb.v_cache.to(dev),
                                          pb.block_table.to(dev), pb.cu_seqlens)
    out = r.out.float().cpu().numpy()
    tot = {"kept": 0, "band": 0, "mismatch_in_band": 0, "mismatch_outside_band": 0, "max_abs_err": 0.0}
    io = co = 0
    Bp, Hqp = w.block_size, w.num_q_heads
    for b, (qb, kb, vb) in enumerate(pb.requests):
        L = qb.shape[0]
        nb = (L + Bp - 1) // Bp
        mask = fp.lists_to_mask(r.kv_idx, r.kv_cnt, Hqp, nb, offset=io, cnt_offset=co)
        qn, kn, vn = qb.float().numpy(), kb.float().numpy(), vb.float().numpy()
        ref = O.select_blocks(qn, kn, vn, Bp, 0.1)
        st_b = _mask_stats(mask, ref.keep, ref.band)
        for key in ("kept", "band", "mismatch_in_band", "mismatch_outside_band"):
            tot[key] += st_b[key]
        t0b = int(pb.cu_seqlens[b])
        pairs = [(int(h), int(I)) for h, I in zip(rng.integers(0, Hqp, 2), rng.integers(0, nb, 2))]
        tot["max_abs_err"] = max(tot["max_abs_err"],
                                 _sampled_error(O, qn, kn, vn, ref, mask, corr, out[t0b:t0b + L], pairs, Bp))
        io += Hqp * nb * (nb + 1) // 2
        co += Hqp * nb
    tot["err_rows"] = "2 random (head, query block) pairs per request"
    res["paged_batch8"] = {"0.1": tot}
    res["seconds"] = round(time.perf_counter() - t0, 1)
    res["tolerance"] = {"bf16": 2e-2, "fp8": 6e-2}
    log(f"bench: parity {res}")
    return res


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return None


def cpu_baseline(q, k, v, B, alpha, corr, head, seconds, oracle_sel=None):
    """The fp64 oracle on the host: full selection, then attention for a
    random sample of (head, query block) pairs under the GPU's mask, in
    batched calls that fill about `seconds`; the rate is scaled by FLOP to the
    whole workload.  cores: the CPUs this process may run on; blas_threads:
    the BLAS pool the oracle's products use."""
    import numpy as np
    import oracle as O
    import block_sparse_long_pooling_amd as fp
    S, Hq, d = q.shape
    nB = (S + B - 1) // B
    qn, kn, vn = q.float().numpy(), k.float().numpy(), v.float().numpy()
    t0 = time.perf_counter()
    sel = O.select_blocks(qn, kn, vn, B, alpha)
    t_sel = time.perf_counter() - t0
    mask = fp.lists_to_mask(head["sel"].kv_idx, head["sel"].kv_cnt, Hq, nB)
    order = [divmod(int(x), nB) for x in np.random.default_rng(0).permutation(Hq * nB)]
    n_full = np.full(nB, B)
    n_full[-1] = S - (nB - 1) * B

    def work(pairs):
        f = 0.0
        for h, I in pairs:
            kept = mask[h, I, :I + 1]
            f += 4.0 * d * n_full[I] * float(n_full[:I + 1][kept].sum())
            if corr:
                f += 4.0 * d * n_full[I] * float((~kept[:I]).sum())
        return f

    # Batched calls of growing size (each call fills an [S, Hq, d] output, so
    # one pair per call would mostly time that fill), the last one sized by
    # the rate measured so far to end near the time budget.
    done, t_att, f_s, n = 0, 0.0, 0.0, 8
    while done < len(order):
        batch = order[done:done + n]
        t1 = time.perf_counter()
        O.sparse_attention(qn, kn, vn, sel, corr, pairs=batch, keep=mask)
        t_att += time.perf_counter() - t1
        f_s += work(batch)
        done += len(batch)
        left = seconds - t_att
        if left <= 0:
            break
        per_pair = t_att / done
        n = int(min(4 * n, max(8, left / per_pair)))
    f_total = head["f_kept"] + head["f_corr"]
    est_total_s = t_sel + t_att * f_total / max(f_s, 1.0)
    cores = len(os.sched_getaffinity(0))
    res = {"value": round(float(f_total / est_total_s / 1e12), 6), "unit": "TFLOP/s",
           "cores": cores, "blas_threads": _blas_threads(), "numpy": np.__version__, "kind": "oracle",
           "sample": f"full fp64 selection ({t_sel:.1f}s) + attention for {done} of {Hq * nB} random "
                     f"(head, query block) pairs in batched calls ({t_att:.1f}s), scaled by FLOP to the "
                     f"whole workload",
           "est_seconds_full": round(float(est_total_s), 1)}
    if oracle_sel is not None:
        oracle_sel.append(sel)
    return res


if __name__ == "__main__":
    main()
