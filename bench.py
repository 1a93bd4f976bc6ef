#!/usr/bin/env python
"""Benchmark of the DSA forward hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
metadata -> lightning-indexer scores (row chunks under a 2 GiB score cap) ->
radix top-K -> sparse attention forward. Workloads 1-5 are packed documents
(plain causal mask); 6 and 7 are split-query / compressed-key workloads
(ratio-causal mask with query causal offsets). Inputs are generated on the
GPU before the timed region and stay resident in HBM.

Prints one JSON line. `value` is the sparse-attention forward throughput in
TFLOP/s (algorithmic FLOP: 2*(D_qk+D_v) per valid slot per head, over the
attention kernel's time measured with HIP events inside the timed steps);
`indexer_topk_rows_per_s` is the second half of the metric; `ms_per_step` is
the whole path. `roofline` describes the dominant kernel; `cpu_baseline` is
the fp64 CPU oracle timed on a bounded sample of the same workload.
`stages_flushed` repeats the stage timings over a few extra steps that each
start after 512 MiB were written, so that the 256 MB MALL holds none of the
step's inputs (the main figures are warm: back-to-back steps).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn fwd TFLOP/s + indexer+topK rows/s at 1 MI355X; % of roofline"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
ATTN_SRC = os.path.join(ROOT, "deepseek_sparse_attention_dsa_amd", "csrc", "sparse_attn.hip")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", type=int, default=2, help="workload 1..10 (default: 2)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--backward", action="store_true",
                   help="also time dsa_sparse_attn_bwd on the forward's outputs (shared latent KV "
                        "workloads), reported as its own stage")
    p.add_argument("--fused", action="store_true",
                   help="one combined indexer + top-K launch instead of score chunks + dsa_topk "
                        "(rows of <= 4096 columns)")
    p.add_argument("--flush-steps", type=int, default=5,
                   help="extra steps, each after writing 512 MiB so that the 256 MB MALL holds "
                        "none of the step's inputs, reported as stages_flushed (0: none)")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="approximate CPU time budget of the oracle baseline")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB (3 times), the "
                        "known-size reference for the FETCH_SIZE / WRITE_SIZE counters")
    p.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR",
                                                            "CAL_FETCH_DIR", "CAL_WRITE_DIR"),
                   help="turn four rocprofv3 --pmc output folders (FETCH_SIZE / WRITE_SIZE of "
                        "this bench, then of --copy-calibration) into "
                        "profiles/traffic_attention_<workload>.json")
    p.add_argument("--calibration-mib", type=int, default=1024,
                   help="size the --copy-calibration run used (for --summarize-traffic)")
    return p.parse_args()


def workload_counts(wl, seq_lens_np):
    """Algorithmic work of one step (what the method must do)."""
    c = {}
    K = wl.topk
    if wl.q_idx is not None:
        sl = seq_lens_np.astype(np.int64)
        pairs = int(sl.sum())  # scored (query, key) pairs: sum of the mask lengths
        c["indexer_flop"] = 2.0 * wl.H_idx * wl.D_idx * pairs
        rd = 4.0 * float(sl[sl > K].sum()) + 8.0 * len(sl)
        wr = (4.0 * K + 4.0) * len(sl)
        c["topk_bytes"] = rd + wr
        c["valid_slots"] = float(np.minimum(sl, K).sum())
    else:
        c["valid_slots"] = float((wl.routes >= 0).sum().item())
    c["attn_flop"] = 2.0 * (wl.D_qk + wl.D_v) * wl.H * c["valid_slots"]
    # bytes of selected KV rows the attention kernel gathers (bf16; a shared
    # latent row serves as both key and value)
    gathered_dims = wl.D_qk + (0 if wl.v is None else wl.D_v)
    c["attn_gathered_bytes"] = 2.0 * gathered_dims * c["valid_slots"]
    return c


def traffic_from_profile(workload_name: str):
    """HBM bytes per attention launch from committed rocprofv3 counters.

    Returns None unless profiles/traffic_<workload>.json exists and was taken
    from the current attention kernel source (sha256 match).
    """
    path = os.path.join(PROFILES, f"traffic_attention_{workload_name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    sha = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
    if rec.get("kernel_source_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def _counter_rows(folder: str, counter: str):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no {counter} rows under {folder}")
    return rows


def summarize_traffic(args):
    """HBM bytes per attention launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch).

    Each counter is scaled by the factor that maps its reading for a plain copy
    of known size (calibration_mib MiB read and written once) onto that size.
    """
    from workloads import CONFIGS
    fetch_dir, write_dir, cal_fetch_dir, cal_write_dir = args.summarize_traffic
    known = args.calibration_mib * 2.0 ** 20
    res = {"workload": CONFIGS[args.config]["name"],
           "kernel_source_sha256": hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest(),
           "calibration_copy_bytes": known}
    for name, folder, cal in (("fetch", fetch_dir, cal_fetch_dir), ("write", write_dir, cal_write_dir)):
        counter = "FETCH_SIZE" if name == "fetch" else "WRITE_SIZE"
        attn = [v for k, v in _counter_rows(folder, counter) if "sparse_attn_kernel" in k]
        copies = [v for k, v in _counter_rows(cal, counter)]
        cal_kib = max(copies)  # the calibration copy is by far the largest dispatch
        factor = known / (cal_kib * 1024.0)
        res[f"{name}_kib_per_launch"] = float(np.mean(attn))
        res[f"{name}_launches"] = len(attn)
        res[f"calibration_{name}_kib"] = cal_kib
        res[f"{name}_scale"] = factor
        res[f"{name}_bytes_per_launch"] = float(np.mean(attn)) * 1024.0 * factor
    res["hbm_bytes_per_launch"] = res["fetch_bytes_per_launch"] + res["write_bytes_per_launch"]
    path = os.path.join(PROFILES, f"traffic_attention_{res['workload']}.json")
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res), flush=True)


def copy_calibration(mib: int):
    import torch
    n = mib * 2 ** 20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4, "repeats": 3}), flush=True)


def cpu_baseline(wl, rs, sl, budget_s):
    """Time the fp64 oracle on a bounded, seeded sample of the workload's rows."""
    from threadpoolctl import threadpool_info

    from oracle import dsa_oracle as O
    from workloads import bf16_to_numpy_bits

    import torch

    f64 = lambda t: O.bf16_bits_to_f64(bf16_to_numpy_bits(t))  # noqa: E731
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    rng = np.random.default_rng(1234)
    T = wl.T
    rs_np, sl_np = rs.cpu().numpy(), sl.cpu().numpy()
    res = {"kind": "oracle", "cores": int(threads), "cpu": platform.processor() or platform.machine()}
    # attention: the oracle on sampled rows with the GPU path's own indices
    kv = f64(wl.kv)
    v = None if wl.v is None else f64(wl.v)
    sink = None if wl.sink is None else wl.sink.cpu().numpy().astype(np.float64)
    idx_all, tl_all = wl.extra["indices"], wl.extra["topk_length"]
    n_att, t_att, flop_att = 0, 0.0, 0.0
    rows_order = rng.permutation(T)
    while t_att < budget_s * 0.5 and n_att < T:
        rows = rows_order[n_att:n_att + 8]
        sel = torch.as_tensor(rows, device=wl.q.device)
        q = f64(wl.q[sel])
        idx = idx_all[sel].cpu().numpy().astype(np.int64)
        tl = None if tl_all is None else tl_all[sel].cpu().numpy()
        t0 = time.perf_counter()
        O.sparse_attention(q, kv, v, idx, tl, sink, wl.scale, d_v=wl.D_v)
        t_att += time.perf_counter() - t0
        valid = (idx >= 0) if tl is None else (np.arange(idx.shape[1])[None, :] < tl[:, None])
        flop_att += 2.0 * (wl.D_qk + wl.D_v) * wl.H * float(valid.sum())
        n_att += len(rows)
    res["value"] = flop_att / t_att / 1e12
    res["unit"] = "TFLOP/s"
    sample = f"attention on {n_att} random rows ({t_att:.1f} s)"
    # indexer + top-K on sampled rows
    if wl.q_idx is not None:
        fp8 = wl.extra.get("fp8")
        if fp8:
            i64 = lambda t: t.cpu().numpy().astype(np.int64)  # noqa: E731
            mx = fp8["scaling"] == "mx"
            k8 = i64(fp8["k8"])
            ks = i64(fp8["k_scale"]) if mx else fp8["k_scale"].cpu().numpy().astype(np.float64)
        else:
            k_idx = f64(wl.k_idx)
        n_idx, t_idx = 0, 0.0
        while t_idx < budget_s * 0.5 and n_idx < T:
            rows = rows_order[n_idx:n_idx + 16]
            sel = torch.as_tensor(rows, device=wl.q_idx.device)
            w = f64(wl.w[sel])
            st, ln = rs_np[rows].astype(np.int64), sl_np[rows].astype(np.int64)
            if fp8:
                q8 = i64(fp8["q8"][sel])
                qs = (i64(fp8["q_scale"][sel]) if mx
                      else fp8["q_scale"][sel].cpu().numpy().astype(np.float64))
                fn = O.indexer_scores_mxfp8 if mx else O.indexer_scores_fp8
                t0 = time.perf_counter()
                sc = fn(q8, qs, k8, ks, w, st, ln, np.arange(len(rows)))
            else:
                q = f64(wl.q_idx[sel])
                t0 = time.perf_counter()
                sc = O.indexer_scores(q, k_idx, w, st, ln, np.arange(len(rows)))
            O.topk(sc, ln, wl.topk, row_starts=st)
            t_idx += time.perf_counter() - t0
            n_idx += len(rows)
        res["indexer_topk_rows_per_s"] = n_idx / t_idx
        sample += f"; indexer+top-K on {n_idx} random rows ({t_idx:.1f} s)"
    res["sample"] = sample
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the DSA forward path here is a single-GPU build "
              "(no collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.summarize_traffic:
        summarize_traffic(args)
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import torch

    import deepseek_sparse_attention_dsa_amd as dsa
    from workloads import CONFIGS, make_config

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    dsa.load_library()
    wl = make_config(args.config, device=dev)
    split = bool(CONFIGS[args.config].get("split"))
    fp8 = wl.extra.get("fp8") if hasattr(wl, "extra") else None
    T, K = wl.T, wl.topk
    # longest score row: the longest document, or the longest key segment
    max_len = max(CONFIGS[args.config]["k_lens"]) if split else max(wl.doc_lens)
    has_indexer = wl.q_idx is not None

    def metadata(row_starts=None, seq_lens=None):
        if split:
            return dsa.dsa_ratio_causal_metadata(wl.cu_seqlens_q, wl.cu_seqlens_k, T, wl.ratio,
                                                 wl.q_causal_offsets, row_starts=row_starts,
                                                 seq_lens=seq_lens)
        return dsa.dsa_packed_metadata(wl.cu_seqlens, T, row_starts=row_starts, seq_lens=seq_lens)

    rs, sl = metadata()
    fused = has_indexer and args.fused
    if fused and max_len > dsa.DSA_FUSED_MAX_COLS:
        raise SystemExit(f"--fused takes rows of at most {dsa.DSA_FUSED_MAX_COLS} columns")
    if fp8:
        fp8_scaling = dsa.DSA_MXFP8 if fp8["scaling"] == "mx" else dsa.DSA_FP8_PER_TOKEN
    rows_per_chunk = dsa.chunk_rows(T, max_len)
    ld = max(4, (max_len + 3) // 4 * 4)
    scores = (None if fused else
              torch.empty((min(rows_per_chunk, T), ld), dtype=torch.float32, device=dev))
    indices = torch.empty((T, K), dtype=torch.int32, device=dev) if has_indexer else wl.routes
    topk_length = torch.empty((T,), dtype=torch.int32, device=dev) if has_indexer else None
    out = torch.empty((T, wl.H, wl.D_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, wl.H), dtype=torch.float32, device=dev)
    max_logits = torch.empty((T, wl.H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    ev = {}

    def step(timed: bool, key: str = "steps"):
        e0 = torch.cuda.Event(enable_timing=True) if timed else None
        e1 = torch.cuda.Event(enable_timing=True) if timed else None
        e2 = torch.cuda.Event(enable_timing=True) if timed else None
        if timed:
            e0.record(stream)
        metadata(rs, sl)
        if has_indexer and fused:
            if fp8:
                dsa.dsa_indexer_topk_fused(fp8["q8"], fp8["k8"], wl.w, rs, sl, K, max_len,
                                           q_scale=fp8["q_scale"], k_scale=fp8["k_scale"],
                                           fp8_scaling=fp8_scaling, indices=indices,
                                           topk_length=topk_length)
            else:
                dsa.dsa_indexer_topk_fused(wl.q_idx, wl.k_idx, wl.w, rs, sl, K, max_len,
                                           indices=indices, topk_length=topk_length)
        elif has_indexer:
            for r0 in range(0, T, rows_per_chunk):
                n = min(rows_per_chunk, T - r0)
                if fp8:
                    dsa.dsa_indexer_fwd_fp8(fp8["q8"], fp8["q_scale"], fp8["k8"], fp8["k_scale"],
                                            wl.w, rs, sl, scaling=fp8_scaling, row_begin=r0,
                                            n_rows=n, scores=scores)
                else:
                    dsa.dsa_indexer_fwd(wl.q_idx, wl.k_idx, wl.w, rs, sl, row_begin=r0,
                                        n_rows=n, scores=scores)
                # plain causal rows never see more than r0 + n keys
                n_cols = max_len if split else min(max_len, r0 + n)
                dsa.dsa_topk(scores[:n], sl[r0:r0 + n], K, row_starts=rs[r0:r0 + n],
                             n_cols=n_cols, indices=indices[r0:r0 + n],
                             topk_length=topk_length[r0:r0 + n])
        if timed:
            e1.record(stream)
        dsa.dsa_sparse_attn_fwd(wl.q, wl.kv, indices, topk_length=topk_length,
                                attn_sink=wl.sink, softmax_scale=wl.scale, v=wl.v, out=out,
                                lse=lse, max_logits=max_logits)
        if timed:
            e2.record(stream)
            ev.setdefault(key, []).append((e0, e1, e2))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if args.flush_steps > 0:
        flush = torch.empty(512 * 2 ** 20 // 4, dtype=torch.float32, device=dev)
        for i in range(args.flush_steps):
            flush.fill_(float(i))  # evicts the step's inputs from the MALL (outside the events)
            step(True, "flushed")
        torch.cuda.synchronize()
        del flush

    idx_ms = [a.elapsed_time(b) for a, b, _ in ev["steps"]]
    att_ms = [b.elapsed_time(c) for _, b, c in ev["steps"]]
    sl_np = sl.cpu().numpy()
    cnt = workload_counts(wl, sl_np)
    att_s = float(np.mean(att_ms)) / 1e3
    attn_tflops = cnt["attn_flop"] / att_s / 1e12
    ms_per_step = wall / args.steps * 1e3

    stages = {"attention": {"ms": float(np.mean(att_ms)), "tflops": attn_tflops,
                            "frac_bf16_peak": attn_tflops / PEAK_BF16_TFLOPS,
                            "algorithmic_flop": cnt["attn_flop"],
                            # gathers are served mostly by L2 and the MALL, so this
                            # rate can exceed the HBM peak
                            "gathered_bytes": cnt["attn_gathered_bytes"],
                            "gather_tb_per_s": cnt["attn_gathered_bytes"] / att_s / 1e12}}
    rows_per_s = None
    if has_indexer:
        idx_s = float(np.mean(idx_ms)) / 1e3
        rows_per_s = T / idx_s
        stages["metadata+indexer+topk"] = {"ms": float(np.mean(idx_ms)), "rows_per_s": rows_per_s,
                                           "indexer_algorithmic_flop": cnt["indexer_flop"],
                                           "topk_algorithmic_bytes": cnt["topk_bytes"],
                                           "chunks": 0 if fused else math.ceil(T / rows_per_chunk),
                                           "combined_launch": fused}

    stages_flushed = None
    if "flushed" in ev:
        f_att = float(np.mean([b.elapsed_time(c) for _, b, c in ev["flushed"]]))
        stages_flushed = {"steps": len(ev["flushed"]), "attention": {
            "ms": f_att, "tflops": cnt["attn_flop"] / f_att / 1e9}}
        if has_indexer:
            f_idx = float(np.mean([a.elapsed_time(b) for a, b, _ in ev["flushed"]]))
            stages_flushed["metadata+indexer+topk"] = {"ms": f_idx, "rows_per_s": T / f_idx * 1e3}

    roofline = {"kernel": "sparse_attn_kernel", "bound": "mfma", "achieved": attn_tflops,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": attn_tflops / PEAK_BF16_TFLOPS,
                "algorithmic_per_launch": cnt["attn_flop"],
                "avg_launch_ms": float(np.mean(att_ms)), "traffic": None}
    tb = traffic_from_profile(CONFIGS[args.config]["name"])
    if tb is not None:
        roofline["traffic"] = tb

    if args.backward and wl.D_v == 512 and wl.v is None:
        g = torch.Generator(device=dev).manual_seed(77)
        dout = (torch.randn(out.shape, generator=g, device=dev) / math.sqrt(wl.D_v)).to(
            torch.bfloat16)
        ws = torch.empty(dsa.dsa_sparse_attn_bwd_workspace_bytes(T, wl.H, wl.kv.shape[0],
                                                                 wl.D_qk, K),
                         dtype=torch.uint8, device=dev)
        dq = torch.empty_like(wl.q)
        dkv = torch.empty((wl.kv.shape[0], wl.D_qk), dtype=torch.bfloat16, device=dev)
        d_sink = torch.empty((wl.H,), dtype=torch.float32, device=dev)

        def bwd():
            dsa.dsa_sparse_attn_bwd(wl.q, wl.kv, indices, out, dout, lse, topk_length=topk_length,
                                    attn_sink=wl.sink, softmax_scale=wl.scale, workspace=ws,
                                    dq=dq, dkv=dkv, d_sink=d_sink)
        for _ in range(max(1, args.warmup)):
            bwd()
        torch.cuda.synchronize()
        bt = []
        for _ in range(max(1, args.steps // 2)):
            b0 = torch.cuda.Event(enable_timing=True)
            b1 = torch.cuda.Event(enable_timing=True)
            b0.record(stream)
            bwd()
            b1.record(stream)
            torch.cuda.synchronize()
            bt.append(b0.elapsed_time(b1))
        bms = float(np.mean(bt))
        # the five products per valid slot and head: s, dP, dq, dk, dv
        bflop = 2.0 * (3 * wl.D_qk + 2 * wl.D_v) * wl.H * cnt["valid_slots"]
        stages["attention_backward"] = {"ms": bms, "tflops": bflop / bms / 1e9,
                                        "frac_bf16_peak": bflop / bms / 1e9 / PEAK_BF16_TFLOPS,
                                        "algorithmic_flop": bflop,
                                        "dkv_row_bytes": 2.0 * wl.D_qk * cnt["valid_slots"]}

    rec = {
        "metric": METRIC, "value": attn_tflops, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": CONFIGS[args.config]["name"], "T": T, "heads": wl.H,
                   "D_qk": wl.D_qk, "D_v": wl.D_v, "topk": K, "indexer_heads": wl.H_idx,
                   "indexer_dim": wl.D_idx, "parallelism": "none"},
        "indexer_topk_rows_per_s": rows_per_s,
        "stages": stages,
        "stages_flushed": stages_flushed,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    rec["config"]["indexer_inputs"] = (
        "bf16" if not fp8 else ("e4m3+e8m0/32" if fp8["scaling"] == "mx" else "e4m3+fp32/token"))
    if split:
        c = CONFIGS[args.config]
        rec["config"].update({"T_kv": wl.T_kv, "ratio": wl.ratio, "q_causal_offsets": c["offsets"],
                              "segments": len(c["q_lens"])})
    else:
        rec["config"]["docs"] = len(wl.doc_lens)
    if not args.no_cpu_baseline:
        wl.extra["indices"] = indices
        wl.extra["topk_length"] = topk_length
        rec["cpu_baseline"] = cpu_baseline(wl, rs, sl, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
