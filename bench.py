#!/usr/bin/env python
"""Benchmark of the DSA forward hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
metadata -> lightning-indexer scores -> radix top-K -> sparse attention
forward. Indexer + top-K run (--path auto) as dsa_indexer_topk_fused with a
candidate buffer for rows longer than 4096 columns (no dense scores),
otherwise as row chunks of scores under a 2 GiB cap followed by dsa_topk.
Workloads 1-5 are packed documents
(plain causal mask); 6 and 7 are split-query / compressed-key workloads
(ratio-causal mask with query causal offsets). Inputs are generated on the
GPU before the timed region and stay resident in HBM.

The default workload is 4, `long_T65536` (one sequence of 65 536 tokens,
64 attention heads over a 576/512 latent KV, a 64 x 128 indexer, top-2048):
the largest single-GPU configuration of the path.

Prints one JSON line. `value` is the sparse-attention forward throughput in
TFLOP/s (algorithmic FLOP: 2*(D_qk+D_v) per valid slot per head, over the
attention kernel's time measured with HIP events inside the timed steps);
`indexer_topk_rows_per_s` is the second half of the metric; `ms_per_step` is
the whole path. Every launch of a timed step is bracketed by its own pair of
HIP events on the launch stream, so each stage (indexer, top-K, or the
combined call; attention) has its own kernel time and roofline in
`rooflines`; `roofline` is the one of
the stage with the most kernel time (the dominant kernel). `cpu_baseline` is
the fp64 CPU oracle, run by a pool of single-threaded worker processes (one
per host core available, at most 16) on a bounded seeded sample of the same
workload. `stages_flushed` repeats the stage timings over a few extra steps
that each start after 512 MiB were written, so that the 256 MB MALL holds
none of the step's inputs (the main figures are warm: back-to-back steps).
`measured_peaks` holds what this device sustains, from the probes of
libdsa_peaks.so run after the timed steps: an MFMA-only loop per MFMA form
(bf16, FP8, MXFP8) and a 16-byte vector copy and read of 1 GiB; each
roofline entry adds `measured_peak` and `frac_of_measured` beside the
published `peak` and `frac`.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import tempfile
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn fwd TFLOP/s + indexer+topK rows/s at 1 MI355X; % of roofline"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "deepseek_sparse_attention_dsa_amd", "csrc")
DEFAULT_CONFIG = 4

# Kernel families of the path: the stage they belong to, the source file they
# are built from, and the substrings that name their dispatches in rocprofv3.
# (The first family whose substring matches takes a dispatch: the candidate
# path's instances come before their plain families.)
KERNELS = {
    "attention": ("sparse_attn.hip", ("sparse_attn_kernel",)),
    "indexer_cand": ("indexer.hip", ("indexer_kernel<128, 2, unsigned short, 2>",)),
    "indexer_rescue": ("indexer.hip", ("indexer_rescue_kernel",)),
    "indexer": ("indexer.hip", ("indexer_kernel<",)),
    "indexer_fp8_cand": ("indexer_fp8.hip", (("indexer_fp8_kernel<", "false, true>"),)),
    "indexer_rescue_fp8": ("indexer_fp8.hip", ("indexer_rescue_fp8_kernel",)),
    "indexer_fp8": ("indexer_fp8.hip", ("indexer_fp8_kernel",)),
    "topk_cand": ("topk.hip", ("topk_radix_kernel<8, 4, true>",)),
    "topk": ("topk.hip", ("topk_radix_kernel", "topk_stream_kernel")),
}
# the kernels of one dsa_indexer_topk_fused call on rows longer than 4096 columns
CAND_FAMILIES = ("indexer_cand", "topk_cand", "indexer_rescue")
CAND_FAMILIES_FP8 = ("indexer_fp8_cand", "topk_cand", "indexer_rescue_fp8")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", type=int, default=DEFAULT_CONFIG,
                   help=f"workload 1..10 (default: {DEFAULT_CONFIG})")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--backward", action="store_true",
                   help="also time dsa_sparse_attn_bwd on the forward's outputs (shared latent KV "
                        "workloads), reported as its own stage")
    p.add_argument("--path", choices=("auto", "chunks", "fused"), default="auto",
                   help="indexer + top-K: score chunks + dsa_topk, or dsa_indexer_topk_fused "
                        "(no dense scores: on chip up to 4096 columns, a candidate buffer "
                        "beyond); auto = fused for rows longer than 4096 columns, else "
                        "chunks")
    p.add_argument("--flush-steps", type=int, default=5,
                   help="extra steps, each after writing 512 MiB so that the 256 MB MALL holds "
                        "none of the step's inputs, reported as stages_flushed (0: none)")
    p.add_argument("--cpu-seconds", type=float, default=20.0,
                   help="approximate wall time of the oracle baseline (both legs)")
    p.add_argument("--cpu-workers", type=int, default=0,
                   help="oracle worker processes (0: the host cores available, at most 16)")
    p.add_argument("--no-peaks", action="store_true",
                   help="skip the measured-peak probes (MFMA loops, HBM copy and read)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB (3 times), the "
                        "known-size reference for the FETCH_SIZE / WRITE_SIZE counters")
    p.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                   help="FETCH_DIR WRITE_DIR CAL_FETCH_DIR CAL_WRITE_DIR [SQ_DIR ...]: turn "
                        "rocprofv3 --pmc output folders of this bench (FETCH_SIZE, WRITE_SIZE, "
                        "then any other counter groups; several runs of one group as "
                        "comma-separated folders) and of --copy-calibration into "
                        "profiles/counters_<workload>.json and .txt")
    p.add_argument("--counter-trace", default="",
                   help="with --summarize-counters: rocprofv3 --kernel-trace --stats folder(s) "
                        "of the same bench command, for the kernels' mean durations")
    p.add_argument("--counter-notes", default="",
                   help="with --summarize-counters: a text file put at the top of the .txt "
                        "summary (the commands that made the runs)")
    p.add_argument("--calibration-mib", type=int, default=1024,
                   help="size the --copy-calibration run used (for --summarize-counters)")
    return p.parse_args()


# ---------------------------------------------------------------------------
# Algorithmic work
# ---------------------------------------------------------------------------

def workload_counts(wl, seq_lens_np):
    """Algorithmic work of one step (what the method must do)."""
    c = {}
    K = wl.topk
    if wl.q_idx is not None:
        sl = seq_lens_np.astype(np.int64)
        pairs = int(sl.sum())  # scored (query, key) pairs: sum of the mask lengths
        c["indexer_flop"] = 2.0 * wl.H_idx * wl.D_idx * pairs
        # top-K reads each score row with more than K columns once, plus the
        # row's start and length, and writes K indices and the row's length
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


# ---------------------------------------------------------------------------
# rocprofv3 counter summaries
# ---------------------------------------------------------------------------

def kernel_source_sha(family: str) -> str:
    """sha256 over the family's source file and every shared header."""
    src, _ = KERNELS[family]
    h = hashlib.sha256()
    for name in [src] + sorted(f for f in os.listdir(CSRC) if f.endswith(".h")):
        h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()


def family_of(kernel_name: str):
    for fam, (_, keys) in KERNELS.items():
        # a key is a substring, or a tuple of substrings that must all occur
        if any(all(p in kernel_name for p in ((k,) if isinstance(k, str) else k))
               for k in keys):
            return fam
    return None


def _counter_rows(folders: str):
    """((run, dispatch id), kernel name, counter, value) from the rocprofv3
    counter CSVs under one folder or several, comma-separated (one run each,
    e.g. the same counters over the bench's two indexer + top-K paths)."""
    import csv
    import glob
    rows = []
    for i, folder in enumerate(folders.split(",")):
        found = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
        if not found:
            raise SystemExit(f"no counter rows under {folder}")
        for f in found:
            for r in csv.DictReader(open(f)):
                rows.append(((i, int(r.get("Dispatch_Id", 0) or 0)), r["Kernel_Name"],
                             r["Counter_Name"], float(r["Counter_Value"])))
    return rows


def _trace_avg_ns(folders: str):
    """{family: mean kernel duration in ns} from rocprofv3 --stats kernel_stats.csv files."""
    import csv
    import glob
    acc = {}
    for folder in folders.split(","):
        for f in glob.glob(os.path.join(folder, "**", "*kernel_stats.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                fam = family_of(r["Name"])
                if fam is not None:
                    tot, n = acc.get(fam, (0.0, 0))
                    acc[fam] = (tot + float(r["TotalDurationNs"]), n + int(r["Calls"]))
    return {f: tot / n for f, (tot, n) in acc.items() if n}


def render_counters(res, notes: str = "") -> str:
    """Text summary of a counters JSON: per kernel family, the HBM bytes per
    launch and the figures derived from the SQ and GRBM counters."""
    out = [notes.rstrip() + "\n"] if notes else []
    out.append(f"workload {res['workload']}; calibration (1 GiB device copy): FETCH_SIZE x "
               f"{res['fetch_scale']:.3f}, WRITE_SIZE x {res['write_scale']:.3f}.")
    out.append("Derived: clock = GRBM_GUI_ACTIVE / 8 XCDs / mean kernel time (kernel trace); "
               "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8); "
               "MFMA FLOP = 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16; co-exec = "
               "SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES; TA busy = TA_TA_BUSY / "
               "(256 CUs x GRBM_GUI_ACTIVE / 8).\n")
    for fam, k in res["kernels"].items():
        out.append(f"{fam}:")
        grbm = k.get("GRBM_GUI_ACTIVE")
        line = []
        if grbm and k.get("kernel_avg_ns"):
            line.append(f"shader clock under load {grbm / 8 / k['kernel_avg_ns']:.2f} GHz "
                        f"(kernel {k['kernel_avg_ns'] / 1e3:.1f} us)")
        if grbm and "SQ_VALU_MFMA_BUSY_CYCLES" in k:
            line.append(f"MFMA busy {100 * k['SQ_VALU_MFMA_BUSY_CYCLES'] / (1024 * grbm / 8):.1f}% "
                        "of SIMD cycles")
        if line:
            out.append("  " + "; ".join(line))
        if k.get("SQ_INSTS_VALU_MFMA_MOPS_BF16"):
            co = k.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0) / max(k["SQ_VALU_MFMA_BUSY_CYCLES"], 1)
            out.append(f"  MFMA FLOP {512 * k['SQ_INSTS_VALU_MFMA_MOPS_BF16']:.3e} per launch; "
                       f"VALU/MFMA co-execution {100 * co:.1f}% of MFMA-busy cycles")
        if "hbm_bytes_per_launch" in k:
            out.append(f"  L2-to-fabric traffic (reads include Infinity Cache hits): FETCH "
                       f"{k['fetch_bytes_per_launch'] / 1e9:.3f} GB + WRITE "
                       f"{k['write_bytes_per_launch'] / 1e9:.3f} GB per launch")
        if grbm and "TA_TA_BUSY" in k:
            out.append(f"  TA busy {100 * k['TA_TA_BUSY'] / (256 * grbm / 8):.1f}%")
        for c in ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "TCP_PENDING_STALL_CYCLES",
                  "TCC_HIT_sum", "TCC_MISS_sum"):
            if c in k:
                out.append(f"  {c} {k[c]:.3e}")
        out.append(f"  kernel source sha256 {k['kernel_source_sha256']}\n")
    return "\n".join(out) + "\n"


def _per_family(rows):
    """{family: {counter: [value per dispatch]}} (values summed over a dispatch's rows)."""
    acc = {}
    for did, kname, cname, val in rows:
        fam = family_of(kname)
        if fam is None:
            continue
        acc.setdefault(fam, {}).setdefault(cname, {}).setdefault(did, 0.0)
        acc[fam][cname][did] += val
    return {f: {c: list(d.values()) for c, d in cs.items()} for f, cs in acc.items()}


def summarize_counters(args):
    """profiles/counters_<workload>.json from rocprofv3 --pmc runs of this bench.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by the factor that
    maps the same counter's reading for a plain copy of known size
    (calibration_mib MiB read and written once) onto that size. Other counters
    are reported as their mean per dispatch.
    """
    from workloads import CONFIGS
    dirs = args.summarize_counters
    if len(dirs) < 4:
        raise SystemExit("--summarize-counters FETCH_DIR WRITE_DIR CAL_FETCH_DIR CAL_WRITE_DIR "
                         "[SQ_DIR ...]")
    fetch_dir, write_dir, cal_fetch_dir, cal_write_dir = dirs[:4]
    known = args.calibration_mib * 2.0 ** 20
    res = {"workload": CONFIGS[args.config]["name"], "calibration_copy_bytes": known,
           "kernels": {}}
    for name, folder, cal in (("fetch", fetch_dir, cal_fetch_dir),
                              ("write", write_dir, cal_write_dir)):
        counter = "FETCH_SIZE" if name == "fetch" else "WRITE_SIZE"
        cal_kib = max(v for _, _, c, v in _counter_rows(cal) if c == counter)
        factor = known / (cal_kib * 1024.0)
        res[f"calibration_{name}_kib"] = cal_kib
        res[f"{name}_scale"] = factor
        for fam, cs in _per_family(_counter_rows(folder)).items():
            vals = cs.get(counter, [])
            if not vals:
                continue
            k = res["kernels"].setdefault(fam, {"kernel_source_sha256": kernel_source_sha(fam)})
            k[f"{name}_kib_per_launch"] = float(np.mean(vals))
            k[f"{name}_launches"] = len(vals)
            k[f"{name}_bytes_per_launch"] = float(np.mean(vals)) * 1024.0 * factor
    for folder in dirs[4:]:
        for fam, cs in _per_family(_counter_rows(folder)).items():
            k = res["kernels"].setdefault(fam, {"kernel_source_sha256": kernel_source_sha(fam)})
            for cname, vals in cs.items():
                k[cname] = float(np.mean(vals))
                k.setdefault("launches", len(vals))
    for fam, k in res["kernels"].items():
        if "fetch_bytes_per_launch" in k and "write_bytes_per_launch" in k:
            k["hbm_bytes_per_launch"] = k["fetch_bytes_per_launch"] + k["write_bytes_per_launch"]
    if args.counter_trace:
        for fam, ns in _trace_avg_ns(args.counter_trace).items():
            if fam in res["kernels"]:
                res["kernels"][fam]["kernel_avg_ns"] = ns
    path = os.path.join(PROFILES, f"counters_{res['workload']}.json")
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    notes = open(args.counter_notes).read() if args.counter_notes else ""
    with open(os.path.join(PROFILES, f"counters_{res['workload']}.txt"), "w") as f:
        f.write(render_counters(res, notes))
    print(json.dumps(res), flush=True)


def traffic_from_profile(workload_name: str, family: str):
    """HBM bytes per launch of a kernel family from committed rocprofv3 counters.

    None unless profiles/counters_<workload>.json holds the family and was
    taken from the current source of its kernels (sha256 match).
    """
    path = os.path.join(PROFILES, f"counters_{workload_name}.json")
    if not os.path.exists(path):
        return None
    k = json.load(open(path)).get("kernels", {}).get(family)
    if not k or k.get("kernel_source_sha256") != kernel_source_sha(family):
        return None
    return k.get("hbm_bytes_per_launch")


def copy_calibration(mib: int):
    import torch
    n = mib * 2 ** 20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4, "repeats": 3}), flush=True)


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a pool of single-threaded processes
# ---------------------------------------------------------------------------

_W = {}  # per-worker arrays (loaded once by the pool initializer)


def _worker_init(folder: str):
    from oracle import dsa_oracle as O
    _W["O"] = O
    for f in os.listdir(folder):
        if f.endswith(".npy"):
            a = np.load(os.path.join(folder, f), mmap_mode="r")
            _W[f[:-4]] = a
    meta = json.load(open(os.path.join(folder, "meta.json")))
    _W["meta"] = meta
    if "kv_bits" in _W:
        _W["kv"] = O.bf16_bits_to_f64(_W["kv_bits"])
        _W["v"] = O.bf16_bits_to_f64(_W["v_bits"]) if "v_bits" in _W else None
    if "k_idx_bits" in _W:
        _W["k_idx"] = O.bf16_bits_to_f64(_W["k_idx_bits"])


def _worker_attention(rows):
    """Oracle attention on sample rows `rows` (indices into the saved sample)."""
    O, m = _W["O"], _W["meta"]
    q = O.bf16_bits_to_f64(np.asarray(_W["q_bits"][rows]))
    idx = np.asarray(_W["att_idx"][rows]).astype(np.int64)
    tl = np.asarray(_W["att_tl"][rows]) if "att_tl" in _W else None
    sink = np.asarray(_W["sink"]) if "sink" in _W else None
    O.sparse_attention(q, _W["kv"], _W["v"], idx, tl, sink, m["scale"], d_v=m["d_v"])
    valid = (idx >= 0) if tl is None else (np.arange(idx.shape[1])[None, :] < tl[:, None])
    return 2.0 * (m["d_qk"] + m["d_v"]) * m["H"] * float(valid.sum())


def _worker_indexer_topk(rows):
    """Oracle indexer scores + top-K on sample rows `rows`."""
    O, m = _W["O"], _W["meta"]
    q = O.bf16_bits_to_f64(np.asarray(_W["qi_bits"][rows]))
    w = O.bf16_bits_to_f64(np.asarray(_W["w_bits"][rows]))
    st = np.asarray(_W["idx_rs"][rows]).astype(np.int64)
    ln = np.asarray(_W["idx_sl"][rows]).astype(np.int64)
    sc = O.indexer_scores(q, _W["k_idx"], w, st, ln, np.arange(len(rows)))
    O.topk(sc, ln, m["topk"], row_starts=st)
    return len(rows)


def _worker_ready(_):
    time.sleep(0.3)  # long enough that each worker takes one of the warm-up tasks
    return os.getpid()


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def _timed_map(pool, fn, chunks):
    t0 = time.perf_counter()
    res = list(pool.map(fn, chunks))
    return time.perf_counter() - t0, res


def cpu_baseline(wl, rs, sl, indices, topk_length, budget_s, workers):
    """Time the fp64 oracle on a bounded, seeded sample of the workload's rows.

    Rows are drawn at random (seed 1234) from the whole workload; each leg
    first runs one row per worker to measure the per-row cost, then a sample
    sized to about budget_s / 2 of wall time, spread over the workers in
    chunks of rows. The rate is sample work over the wall time of that map.
    """
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    from workloads import bf16_to_numpy_bits

    import torch

    P = workers or min(16, len(os.sched_getaffinity(0)))
    T = wl.T
    rng = np.random.default_rng(1234)
    order = rng.permutation(T)
    n_take = min(T, 4096)
    take = np.sort(order[:n_take])
    sel = torch.as_tensor(take, device=wl.q.device)
    folder = tempfile.mkdtemp(prefix="dsa_oracle_", dir="/tmp")
    meta = {"scale": float(wl.scale), "d_v": int(wl.D_v), "d_qk": int(wl.D_qk), "H": int(wl.H),
            "topk": int(wl.topk)}
    json.dump(meta, open(os.path.join(folder, "meta.json"), "w"))
    save = lambda n, a: np.save(os.path.join(folder, n + ".npy"), a)  # noqa: E731
    save("q_bits", bf16_to_numpy_bits(wl.q[sel]))
    save("kv_bits", bf16_to_numpy_bits(wl.kv))
    if wl.v is not None:
        save("v_bits", bf16_to_numpy_bits(wl.v))
    save("att_idx", indices[sel].cpu().numpy())
    if topk_length is not None:
        save("att_tl", topk_length[sel].cpu().numpy())
    if wl.sink is not None:
        save("sink", wl.sink.cpu().numpy().astype(np.float64))
    has_idx = wl.q_idx is not None
    if has_idx:
        save("qi_bits", bf16_to_numpy_bits(wl.q_idx[sel]))
        save("k_idx_bits", bf16_to_numpy_bits(wl.k_idx))
        save("w_bits", bf16_to_numpy_bits(wl.w[sel]))
        save("idx_rs", rs[sel].cpu().numpy())
        save("idx_sl", sl[sel].cpu().numpy())
    # shuffled positions into the saved sample, so every chunk is a random draw
    pos = rng.permutation(n_take)

    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                           "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    res = {"kind": "oracle", "cores": P, "cpu": _cpu_model(),
           "threads_per_worker": 1, "host_cores_visible": len(os.sched_getaffinity(0))}
    try:
        # spawned workers (a fresh interpreter each: nothing of this process's GPU
        # state is inherited); a worker that dies raises instead of hanging
        with ProcessPoolExecutor(P, mp_context=mp.get_context("spawn"), initializer=_worker_init,
                                 initargs=(folder,)) as pool:
            # start and initialise every worker before anything is timed
            pids = set()
            for _ in range(4):
                pids |= set(pool.map(_worker_ready, range(P)))
                if len(pids) >= P:
                    break

            def leg(fn, start):
                # calibration: one row per worker
                cal = [pos[(start + i) % n_take: (start + i) % n_take + 1] for i in range(P)]
                t_cal, _ = _timed_map(pool, fn, cal)
                per_row = max(t_cal, 1e-3)  # one row per worker, in parallel
                n_rows = int(min(n_take, max(P, P * (budget_s / 2.0) / per_row)))
                chunk = max(1, n_rows // (4 * P))
                rows = [pos[(start + i) % n_take] for i in range(n_rows)]
                chunks = [np.sort(np.array(rows[i:i + chunk])) for i in range(0, n_rows, chunk)]
                t, out = _timed_map(pool, fn, chunks)
                return n_rows, t, out

            n_att, t_att, flops = leg(_worker_attention, 0)
            res["value"] = float(sum(flops)) / t_att / 1e12
            res["unit"] = "TFLOP/s"
            sample = (f"subset: attention on {n_att} random rows of {T} ({t_att:.1f} s wall on "
                      f"{P} processes)")
            if has_idx:
                n_idx, t_idx, _ = leg(_worker_indexer_topk, n_take // 2)
                res["indexer_topk_rows_per_s"] = n_idx / t_idx
                sample += (f"; indexer+top-K on {n_idx} random rows of {T} ({t_idx:.1f} s wall "
                           f"on {P} processes)")
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
        for f in os.listdir(folder):
            os.remove(os.path.join(folder, f))
        os.rmdir(folder)
    res["sample"] = sample
    return res


# ---------------------------------------------------------------------------
# The timed path
# ---------------------------------------------------------------------------

def measure_peaks(stream, reps: int = 5):
    """Rates this device sustains: MFMA-only loops (bf16, FP8, MXFP8; 4 waves per
    SIMD, register operands) and a 1 GiB 16-byte vector copy and read, each the
    median of `reps` launches after one warm-up, timed with events on `stream`."""
    import ctypes

    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "deepseek_sparse_attention_dsa_amd", "libdsa_peaks.so"))
    lib.dsa_peak_mfma_flop.restype = ctypes.c_double
    lib.dsa_peak_mfma_flop.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32]
    lib.dsa_peak_mfma.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                  ctypes.c_void_p]
    lib.dsa_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                  ctypes.c_int32, ctypes.c_void_p]
    lib.dsa_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_void_p, ctypes.c_void_p]
    threads = lib.dsa_peak_threads_per_block()
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    sp = ctypes.c_void_p(stream.cuda_stream)

    def timed(fn):
        fn()
        ms = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            rc = fn()
            b.record(stream)
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"peak probe failed ({rc})")
            ms.append(a.elapsed_time(b))
        return float(np.median(ms))

    res = {"compute_units": n_cu}
    blocks = 4 * n_cu  # four workgroups of four waves per CU: four waves per SIMD
    sink = torch.empty((blocks * threads,), dtype=torch.float32, device="cuda:0")
    for name, kind, iters in (("bf16", 0, 4000), ("fp8", 1, 2000), ("mxfp8", 2, 2000)):
        ms = timed(lambda: lib.dsa_peak_mfma(kind, iters, blocks, ctypes.c_void_p(sink.data_ptr()),
                                             sp))
        res[f"{name}_mfma_tflops"] = lib.dsa_peak_mfma_flop(kind, iters, blocks) / ms / 1e9
    del sink
    nbytes = 1 << 30
    src = torch.ones((nbytes // 4,), dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    cblocks = 4 * n_cu
    wsink = torch.empty((cblocks * threads,), dtype=torch.int32, device="cuda:0")
    ms = timed(lambda: lib.dsa_peak_copy(ctypes.c_void_p(src.data_ptr()),
                                         ctypes.c_void_p(dst.data_ptr()), nbytes, cblocks, sp))
    res["hbm_copy_gbs"] = 2.0 * nbytes / ms / 1e6
    ms = timed(lambda: lib.dsa_peak_read(ctypes.c_void_p(src.data_ptr()), nbytes, cblocks,
                                         ctypes.c_void_p(wsink.data_ptr()), sp))
    res["hbm_read_gbs"] = nbytes / ms / 1e6
    del src, dst, wsink
    return res


def add_measured(entry, peaks, mx=False):
    """measured_peak / frac_of_measured of a roofline entry (its own MFMA form or
    the HBM copy rate)."""
    if not peaks:
        return
    if entry["unit"] == "GB/s":
        m = peaks["hbm_copy_gbs"]
    elif entry["peak"] == PEAK_FP8_TFLOPS:
        m = peaks["mxfp8_mfma_tflops" if mx else "fp8_mfma_tflops"]
    else:
        m = peaks["bf16_mfma_tflops"]
    entry["measured_peak"] = m
    entry["frac_of_measured"] = entry["achieved"] / m


def roofline_entry(kernel, bound, algorithmic_total, launches, kernel_ms_total, peak, unit,
                   traffic):
    """Roofline of one kernel family over one step: achieved = algorithmic work per
    launch / average launch duration (= step total / step kernel time)."""
    per_launch = algorithmic_total / max(launches, 1)
    avg_ms = kernel_ms_total / max(launches, 1)
    scale = 1e12 if unit == "TFLOP/s" else 1e9
    achieved = per_launch / (avg_ms / 1e3) / scale
    return {"kernel": kernel, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
            "frac": achieved / peak, "algorithmic_per_launch": per_launch,
            "launches_per_step": launches, "avg_launch_ms": avg_ms, "traffic": traffic}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the DSA forward path here is a single-GPU build "
              "(no collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.summarize_counters:
        summarize_counters(args)
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
    wname = CONFIGS[args.config]["name"]
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
    long_rows = max_len > dsa.DSA_FUSED_MAX_COLS
    fused = has_indexer and (args.path == "fused" or (args.path == "auto" and long_rows))
    long_fused = fused and long_rows
    cand = None
    if long_fused:  # allocated once, outside the timed steps
        cand = torch.empty((dsa.dsa_indexer_topk_cand_buffer_size(T, max_len, K),),
                           dtype=torch.float32, device=dev)
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
    idx_family = "indexer_fp8" if fp8 else "indexer"

    # (stage, start event, end event) per launch, per timed step
    records = {}

    def step(timed: bool, key: str = "steps"):
        evs = []

        def run(stage, fn):
            if timed:
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn()
                b.record(stream)
                evs.append((stage, a, b))
            else:
                fn()

        run("metadata", lambda: metadata(rs, sl))
        if has_indexer and fused:
            if fp8:
                run("indexer_topk_fused", lambda: dsa.dsa_indexer_topk_fused(
                    fp8["q8"], fp8["k8"], wl.w, rs, sl, K, max_len, q_scale=fp8["q_scale"],
                    k_scale=fp8["k_scale"], fp8_scaling=fp8_scaling, indices=indices,
                    topk_length=topk_length, cand_buffer=cand))
            else:
                run("indexer_topk_fused", lambda: dsa.dsa_indexer_topk_fused(
                    wl.q_idx, wl.k_idx, wl.w, rs, sl, K, max_len, indices=indices,
                    topk_length=topk_length, cand_buffer=cand))
        elif has_indexer:
            for r0 in range(0, T, rows_per_chunk):
                n = min(rows_per_chunk, T - r0)
                if fp8:
                    run("indexer", lambda: dsa.dsa_indexer_fwd_fp8(
                        fp8["q8"], fp8["q_scale"], fp8["k8"], fp8["k_scale"], wl.w, rs, sl,
                        scaling=fp8_scaling, row_begin=r0, n_rows=n, scores=scores))
                else:
                    run("indexer", lambda: dsa.dsa_indexer_fwd(
                        wl.q_idx, wl.k_idx, wl.w, rs, sl, row_begin=r0, n_rows=n, scores=scores))
                # plain causal rows never see more than r0 + n keys
                n_cols = max_len if split else min(max_len, r0 + n)
                run("topk", lambda: dsa.dsa_topk(
                    scores[:n], sl[r0:r0 + n], K, row_starts=rs[r0:r0 + n], n_cols=n_cols,
                    indices=indices[r0:r0 + n], topk_length=topk_length[r0:r0 + n]))
        run("attention", lambda: dsa.dsa_sparse_attn_fwd(
            wl.q, wl.kv, indices, topk_length=topk_length, attn_sink=wl.sink,
            softmax_scale=wl.scale, v=wl.v, out=out, lse=lse, max_logits=max_logits))
        if timed:
            records.setdefault(key, []).append(evs)

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

    def stage_times(key):
        """Mean per step of {stage: (kernel ms, launches)} and of the indexer-side span."""
        per = {}
        span = []
        for evs in records[key]:
            tot = {}
            for stage, a, b in evs:
                ms, n = tot.get(stage, (0.0, 0))
                tot[stage] = (ms + a.elapsed_time(b), n + 1)
            for stage, v in tot.items():
                per.setdefault(stage, []).append(v)
            # metadata + indexer + top-K, from the first launch to the last before attention
            idx_evs = [(a, b) for s, a, b in evs if s != "attention"]
            span.append(idx_evs[0][0].elapsed_time(idx_evs[-1][1]))
        mean = {s: (float(np.mean([v[0] for v in vs])), vs[0][1]) for s, vs in per.items()}
        return mean, float(np.mean(span))

    st, idx_span_ms = stage_times("steps")
    sl_np = sl.cpu().numpy()
    cnt = workload_counts(wl, sl_np)
    att_ms = st["attention"][0]
    att_s = att_ms / 1e3
    attn_tflops = cnt["attn_flop"] / att_s / 1e12
    ms_per_step = wall / args.steps * 1e3

    stages = {"attention": {"ms": att_ms, "tflops": attn_tflops,
                            "frac_bf16_peak": attn_tflops / PEAK_BF16_TFLOPS,
                            "algorithmic_flop": cnt["attn_flop"],
                            # gathers are served mostly by L2 and the MALL, so this
                            # rate can exceed the HBM peak
                            "gathered_bytes": cnt["attn_gathered_bytes"],
                            "gather_tb_per_s": cnt["attn_gathered_bytes"] / att_s / 1e12}}
    rooflines = {"attention": roofline_entry(
        "sparse_attn_kernel", "mfma", cnt["attn_flop"], 1, att_ms, PEAK_BF16_TFLOPS, "TFLOP/s",
        traffic_from_profile(wname, "attention"))}
    rows_per_s = None
    if has_indexer:
        rows_per_s = T / (idx_span_ms / 1e3)
        stages["metadata+indexer+topk"] = {
            "ms": idx_span_ms, "rows_per_s": rows_per_s,
            "metadata_ms": st["metadata"][0],
            "indexer_algorithmic_flop": cnt["indexer_flop"],
            "topk_algorithmic_bytes": cnt["topk_bytes"],
            "chunks": 0 if fused else math.ceil(T / rows_per_chunk), "combined_launch": fused}
        idx_peak = PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS
        if fused:
            ms, n = st["indexer_topk_fused"]
            stages["indexer_topk_fused"] = {"ms": ms, "calls": n,
                                            "candidate_buffer": long_fused}
            if long_fused:
                stages["indexer_topk_fused"]["rows_rescued"] = int(
                    cand[:1].view(torch.int32).item())
            traffic = None
            if long_fused:
                parts = [traffic_from_profile(wname, f)
                         for f in (CAND_FAMILIES_FP8 if fp8 else CAND_FAMILIES)]
                traffic = None if any(v is None for v in parts) else float(sum(parts))
            kname = "indexer_fp8_kernel" if fp8 else "indexer_kernel"
            rooflines["indexer_topk_fused"] = roofline_entry(
                f"{kname} (candidate mode) + topk_radix_kernel (candidates) + "
                f"{kname.replace('indexer_', 'indexer_rescue_', 1)}" if long_fused
                else f"{kname} (combined with top-K)",
                "mfma", cnt["indexer_flop"], n, ms, idx_peak, "TFLOP/s", traffic)
        else:
            ims, n_i = st["indexer"]
            tms, n_t = st["topk"]
            stages["indexer"] = {"ms": ims, "launches": n_i,
                                 "tflops": cnt["indexer_flop"] / (ims / 1e3) / 1e12}
            stages["topk"] = {"ms": tms, "launches": n_t,
                              "gb_per_s": cnt["topk_bytes"] / (tms / 1e3) / 1e9}
            rooflines["indexer"] = roofline_entry(
                "indexer_fp8_kernel" if fp8 else "indexer_kernel", "mfma", cnt["indexer_flop"],
                n_i, ims, idx_peak, "TFLOP/s", traffic_from_profile(wname, idx_family))
            rooflines["topk"] = roofline_entry(
                "topk_radix_kernel + topk_stream_kernel", "hbm", cnt["topk_bytes"], n_t, tms,
                PEAK_HBM_GBS, "GB/s", traffic_from_profile(wname, "topk"))

    stages_flushed = None
    if "flushed" in records:
        fst, f_span = stage_times("flushed")
        f_att = fst["attention"][0]
        stages_flushed = {"steps": len(records["flushed"]), "attention": {
            "ms": f_att, "tflops": cnt["attn_flop"] / f_att / 1e9}}
        if has_indexer:
            stages_flushed["metadata+indexer+topk"] = {"ms": f_span,
                                                       "rows_per_s": T / f_span * 1e3}
            if "indexer" in fst:
                stages_flushed["indexer"] = {"ms": fst["indexer"][0]}
                stages_flushed["topk"] = {"ms": fst["topk"][0]}

    peaks = None if args.no_peaks else measure_peaks(stream)
    for e in rooflines.values():
        add_measured(e, peaks, mx=bool(fp8) and fp8["scaling"] == "mx")

    # the dominant kernel: the stage with the most kernel time per step
    dominant = max(rooflines, key=lambda s: rooflines[s]["avg_launch_ms"] *
                   rooflines[s]["launches_per_step"])
    roofline = dict(rooflines[dominant])
    roofline["stage"] = dominant

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
        tiles = dsa.dsa_sparse_attn_bwd_kv_tiles(wl.kv.shape[0], K)
        stages["attention_backward"] = {"ms": bms, "tflops": bflop / bms / 1e9,
                                        "frac_bf16_peak": bflop / bms / 1e9 / PEAK_BF16_TFLOPS,
                                        "algorithmic_flop": bflop,
                                        "dkv_scheme": "kv_tiles" if tiles else "per_slot_rows"}
        if not tiles:  # bf16 dkv rows written and read back once per valid slot
            stages["attention_backward"]["dkv_row_bytes"] = 2.0 * wl.D_qk * cnt["valid_slots"]

    rec = {
        "metric": METRIC, "value": attn_tflops, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wname, "T": T, "heads": wl.H,
                   "D_qk": wl.D_qk, "D_v": wl.D_v, "topk": K, "indexer_heads": wl.H_idx,
                   "indexer_dim": wl.D_idx, "parallelism": "none"},
        "indexer_topk_rows_per_s": rows_per_s,
        "stages": stages,
        "stages_flushed": stages_flushed,
        "roofline": roofline,
        "rooflines": rooflines,
        "measured_peaks": peaks,
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
        rec["cpu_baseline"] = cpu_baseline(wl, rs, sl, indices, topk_length, args.cpu_seconds,
                                           args.cpu_workers)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
