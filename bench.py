#!/usr/bin/env python3
"""Throughput of the fused norm-rope-cache hot path on one MI355X.

One step = one call of the entry point over one batch of the workload
(default: the paged prefill batch B=8, S=4096, D=576 into PA_BNSD caches
[8192, 128, 1, 512/64] bf16). Inputs are synthetic and seeded (gen/), already
resident in HBM when the timed region starts.

Measurement:
  * R independent buffer sets (inputs and caches) are rotated so that the
    touched bytes of R consecutive steps exceed the 256 MB Infinity Cache;
    every step therefore reads its inputs from HBM;
  * one eager launch per buffer set first (setup: loads the library, checks
    every argument set and measures the host's cost of a launch call); then
    exactly W warm-up and exactly K timed launches, continuing the rotation;
  * the launches are enqueued behind a spin kernel that lasts at least twice
    their total host cost, so they are all submitted before the first one
    starts and run back to back; HIP events on the launch stream bracket the
    K timed launches: ms_per_step = elapsed / K, value = tokens / step time,
    and the kernel's average launch duration is the same elapsed / K (one
    launch per step); the line says whether the host did finish enqueuing
    first (--timing graph replays two HIP graphs instead);
  * roofline: algorithmic bytes (or flops) per launch / average launch
    duration, against the MI355X HBM3E peak of 8 TB/s (or the bf16 dense
    matrix peak); rocprof_kernel_us repeats the per-dispatch duration
    percentiles of the committed rocprofv3 trace of the same kernel code;
  * traffic: HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs,
    scaled by the same counters' reading on a plain copy of known size, read
    from profiles/traffic_<workload>.json and reported only if the kernel
    sources are unchanged since the counters were taken (else null);
  * context (same harness, after the timed region): p10 / p50 / p90 of up
    to 200 of the same launches each timed alone between its own events, the
    average step of an empty kernel (one workgroup, and the workload's grid)
    and of a plain device copy moving the same bytes as one launch, each in
    a graph of K launches like the timed region;
  * cpu_baseline: the CPU oracle on the host, on the same batch, about 8 s
    on one thread and 8 s on all the threads it uses, with the CPU model.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "tokens/s and achieved HBM GB/s (% of MI355X peak), fused norm-rope-cache"
HBM_PEAK_GBPS = 8000.0
_COMMON_SOURCES = ["latent_attention_kv_amd/csrc/device_common.hpp",
                   "latent_attention_kv_amd/csrc/kvrc_launch.hpp",
                   "latent_attention_kv_amd/_build.py"]
KERNEL_SOURCES = {
    "kvrc": ["latent_attention_kv_amd/csrc/norm_rope_cache.hip"] + _COMMON_SOURCES,
    "qsa": ["latent_attention_kv_amd/csrc/qsa_prepare.hip"] + _COMMON_SOURCES,
    "mla": ["latent_attention_kv_amd/csrc/mla_kv_head.hip"] + _COMMON_SOURCES,
    "sel": ["latent_attention_kv_amd/csrc/qsa_select.hip"] + _COMMON_SOURCES,
}
KERNEL_NAME = {"kvrc": "norm_rope_cache", "qsa": "qsa_prepare", "mla": "mla_kv_head_kernel",
               "sel": "qsa_select"}

WORKLOAD_TEXT = {
    "prefill_paged": "paged prefill: B=8, S=4096 (32768 tokens), kv [8,1,4096,576] bf16 "
                     "(Dv=512 RMSNorm, Dk=64 interleaved RoPE), PA_BNSD caches "
                     "[8192,128,1,512] + [8192,128,1,64] bf16, 32 blocks per sequence",
    "decode_paged": "paged decode: B=256, S=1, D=576 bf16, caches [4096,128,1,512/64] bf16, "
                    "unique random slots, 5% skipped (-1)",
    "quant_paged": "paged int8 ckv cache: B=64, S=1024, D=576 bf16 (sigma 2), ckv int8 "
                   "[4096,128,1,512] + fp32 scale [4096,128,1], k bf16 [4096,128,1,64]",
    "quant_fp8_paged": "paged FLOAT8 E4M3FN ckv cache: B=64, S=1024, D=576 bf16 (sigma 2), "
                       "ckv E4M3FN [4096,128,1,512] + fp32 scale [4096,128,1], "
                       "k bf16 [4096,128,1,64]",
    "norm_tiny": "Norm cache mode: B=2, S=16, D=576, caches [2,1,32,d] bf16",
    "prefill_paged_blk": "paged prefill, block-indexed (PA_BLK_BNSD): B=8, S=4096 (32768 "
                         "tokens), D=576 bf16, one index entry per 128-token chunk, caches "
                         "[8192,128,1,512] + [8192,128,1,64] bf16",
    "qsa": "QSAPrepare block keys: N=32, L=2048, Di=128, Dr=64, key_block_size=64",
    "mla_kv_head": "MLA kv-path head: T=32768 tokens (B=8, S=4096), x [32768,7168] bf16 times "
                   "the fused projection [576,7168] bf16 (random init) on the matrix cores, "
                   "alpha_kv 0.875, RMSNorm + RoPE, PA_BNSD caches [8192,128,1,512/64] bf16",
    "mla_kv_head_int8": "MLA kv-path head as mla_kv_head (T=32768, He=7168) into an int8 ckv "
                        "cache [8192,128,1,512] + fp32 scale [8192,128,1] (RowMax/127), k "
                        "cache bf16 [8192,128,1,64]",
    "mla_kv_head_fp8": "MLA kv-path head as mla_kv_head (T=32768, He=7168) into a FLOAT8 "
                       "E4M3FN ckv cache [8192,128,1,512] + fp32 scale [8192,128,1] "
                       "(RowMax/448), k cache bf16 [8192,128,1,64]",
    "qsa_select": "block selection: N=128 sequences x 1 query token, H=64 heads, Di=128, block "
                  "keys [128,256,128] bf16 (key_length U[4096,16384), key_block_size 64), "
                  "selection blocks of 2 key blocks, top 16",
}
MFMA_BF16_PEAK_TFLOPS = 2500.0


def kernel_family(workload: str) -> str:
    if workload.startswith("mla_kv_head"):
        return "mla"
    return {"qsa": "qsa", "qsa_select": "sel"}.get(workload, "kvrc")


def _code_only(rel: str, text: str) -> str:
    """The source without comments and blank lines (C++: // and /* */;
    Python: whole-line # comments), so that editing a comment does not
    disown counters taken on the same code."""
    if rel.endswith(".py"):
        lines = [ln.rstrip() for ln in text.splitlines() if not ln.lstrip().startswith("#")]
    else:
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
    return "\n".join(ln for ln in lines if ln.strip())


def source_hash(workload: str) -> str:
    """Hash of the code that builds the workload's kernel (counters taken on
    another version of it are not reported)."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel_family(workload)]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(rel, f.read()).encode())
    return h.hexdigest()[:16]


def algorithmic_flops(case) -> int:
    """Multiply-add work of the projection: 2 * T * 576 * He (MLA head only)."""
    return 2 * case["T"] * 576 * case["He"] if case.get("mode") == "mla_paged" else 0


def algorithmic_bytes(case) -> tuple[int, int]:
    """(bytes per launch, tokens per launch) the method must move."""
    import gen
    if "block_keys" in case and "query" in case:
        total = 0
        kl = case["key_length"]
        for n in range(case["N"]):
            nb = int(kl[n % len(kl)]) // case["kbs"]
            total += case["H"] * case["Di"] * 2 + nb * case["Di"] * 2 + 8
            total += case["Jcap"] * 4 + case["topk"] * 4
        return total, case["N"]
    if case.get("mode") == "mla_paged":
        T, He = case["T"], case["He"]
        written = int((case["slot_mapping"] >= 0).sum())
        ckv_row = 1024 if case.get("ckv_dtype", "bf16") == "bf16" else 512 + 4
        return (T * He * 2 + 576 * He * 2 + T * (2 * 2 * 64 + 8) + written * (ckv_row + 128)
                + 1024, T)
    if "raw_index_keys" in case:
        N, L, Di, Dr, kbs = case["N"], case["L"], case["Di"], case["Dr"], case["kbs"]
        total = 0
        for n in range(N):
            K = int(case["key_length"][n % len(case["key_length"])])
            P = K - L
            r, r2 = P % kbs, K % kbs
            nb = K // kbs - P // kbs
            total += L * Di * 2 + (r if nb else 0) * Di * 2      # new rows + carried rows read
            total += nb * (2 * Dr * 4 + Di * 2)                   # first-token rope row + key out
            total += r2 * Di * 2 * 2 + (2 * Dr * 4 * 2 if r2 else 0)  # carry copy in/out
            total += 8                                            # key_length
        return total + Di * 2, N * L
    T = case["B"] * case["S"]
    per = gen.kvrc_bytes_per_written_token(case["Dv"], case["Dk"], case["ckv_dtype"])
    if case["mode"] == "paged_blk":
        # one 8-byte entry per chunk instead of one per token
        S, bs = case["S"], case["block_size"]
        chunks = -(-S // bs)
        entries = case["block_index"].reshape(case["B"], chunks)
        written = sum(min(bs, S - c * bs) for b in range(case["B"]) for c in range(chunks)
                      if entries[b, c] >= 0)
        return written * (per - 8) + entries.size * 8 + 2 * case["Dv"], T
    idx = case["slot_mapping"] if case["mode"] == "paged" else case["index"].reshape(-1)
    written = int((idx >= 0).sum())
    return written * per + (T - written) * 8 + 2 * case["Dv"], T


def touched_bytes(case) -> int:
    return algorithmic_bytes(case)[0]


def build_sets(case, R, dev):
    """R independent device copies of the inputs and caches."""
    import numpy as np
    import torch

    def dbf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    def dt(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    sets = []
    if "block_keys" in case and "query" in case:
        base = dict(q=dbf(case["query"]), keys=dbf(case["block_keys"]), kl=dt(case["key_length"]))
        for i in range(R):
            s = {k: (v.clone() if i else v) for k, v in base.items()}
            s["scores"] = torch.zeros(case["N"], case["Jcap"], dtype=torch.float32, device=dev)
            s["idx"] = torch.zeros(case["N"], case["topk"], dtype=torch.int32, device=dev)
            sets.append(s)
        return sets
    if case.get("mode") == "mla_paged":
        import latent_attention_kv_amd as kvlib
        base = dict(x=dbf(case["x"]), w=dbf(case["w"]), gamma=dbf(case["gamma"]),
                    cos=dbf(case["cos"]), sin=dbf(case["sin"]), idx=dt(case["slot_mapping"]))
        # the launches run in order on one stream: one zeroed workspace serves all
        ws = torch.zeros(kvlib.kvrc_mla_kv_head_workspace_bytes(case["x"].shape[0]),
                         dtype=torch.uint8, device=dev)
        for i in range(R):
            s = {k: (v.clone() if i else v) for k, v in base.items()}
            s["ws"] = ws
            s.update(_cache_tensors(case, dev))
            sets.append(s)
        return sets
    if "raw_index_keys" in case:
        base = dict(raw=dbf(case["raw_index_keys"]), kl=dt(case["key_length"]),
                    rc=dt(case["rope_cos"]), rs=dt(case["rope_sin"]), w=dbf(case["k_norm_weight"]),
                    praw=dbf(case["past_incomplete_raw_keys"]),
                    prope=dt(case["past_incomplete_rope"]))
        for _ in range(R):
            s = {k: v.clone() for k, v in base.items()}
            s["bk"] = dbf(case["caches"]["block_keys"].numpy())
            s["nraw"] = torch.empty_like(s["praw"])
            s["nrope"] = torch.empty_like(s["prope"])
            sets.append(s)
        return sets
    idx_name = {"paged": "slot_mapping", "paged_blk": "block_index"}.get(case["mode"], "index")
    base = dict(kv=dbf(case["kv"]), gamma=dbf(case["gamma"]), cos=dbf(case["cos"]),
                sin=dbf(case["sin"]), idx=dt(case[idx_name]))
    for _ in range(R):
        s = {k: v.clone() for k, v in base.items()}
        s.update(_cache_tensors(case, dev))
        sets.append(s)
    return sets


def _cache_tensors(case, dev):
    """Fresh device caches of the case, filled with their sentinels."""
    import numpy as np
    import torch
    out = {}
    for name, spec in case["caches"].items():
        if spec.dtype == np.uint16:
            fill = int(np.array([spec.fill], dtype=np.uint16).view(np.int16)[0])
            out[name] = torch.full(spec.shape, fill, dtype=torch.int16,
                                   device=dev).view(torch.bfloat16)
        else:
            tdt = {np.dtype(np.int8): torch.int8, np.dtype(np.uint8): torch.uint8,
                   np.dtype(np.float32): torch.float32}[spec.dtype]
            out[name] = torch.full(spec.shape, spec.fill, dtype=tdt, device=dev)
    return out


def launch(case, s):
    import latent_attention_kv_amd as k
    if "block_keys" in case and "query" in case:
        k.qsa_select_topk(s["q"], s["keys"], s["kl"], s["scores"], s["idx"],
                          key_block_size=case["kbs"], sel_ratio=case["sel_ratio"],
                          cmp_ratio=case["cmp_ratio"], scale=case["scale"])
    elif case.get("mode") == "mla_paged":
        k.kvrc_mla_kv_head_paged(s["x"], s["w"], s["gamma"], s["cos"], s["sin"], s["idx"],
                                 s["k_cache"], s["ckv_cache"], s.get("ckv_scale"),
                                 workspace=s["ws"], alpha_kv=case["alpha"], eps=case["eps"])
    elif "raw_index_keys" in case:
        k.qsa_prepare(s["raw"], s["bk"], s["kl"], s["rc"], s["rs"], s["w"], s["praw"], s["prope"],
                      s["nraw"], s["nrope"], key_block_size=case["kbs"], eps=case["eps"])
    elif case["mode"] == "paged":
        k.kvrc_paged_norm_rope_cache(s["kv"], s["gamma"], s["cos"], s["sin"], s["idx"],
                                     s["k_cache"], s["ckv_cache"], s.get("ckv_scale"),
                                     eps=case["eps"])
    elif case["mode"] == "paged_blk":
        k.kvrc_paged_blk_norm_rope_cache(s["kv"], s["gamma"], s["cos"], s["sin"], s["idx"],
                                         s["k_cache"], s["ckv_cache"], s.get("ckv_scale"),
                                         eps=case["eps"])
    else:
        k.kvrc_norm_rope_cache(s["kv"], s["gamma"], s["cos"], s["sin"], s["idx"], s["k_cache"],
                               s["ckv_cache"], s.get("ckv_scale"), eps=case["eps"])


def _oracle_run(case, threads, seconds):
    """Run the oracle, as it is, on the workload until about `seconds` of
    oracle time have passed: (runs, busy seconds, tokens per run, what ran).
    `threads` is the oracle's OpenMP thread count (numpy's BLAS threads for
    the float64 oracles). Caches are allocated once, outside the timing; each
    run rewrites the same rows with the same values."""
    import oracle
    n, busy = 0, 0.0

    def loop(fn):
        nonlocal n, busy
        while busy < seconds or n == 0:
            s0 = time.perf_counter()
            fn()
            busy += time.perf_counter() - s0
            n += 1

    if "block_keys" in case and "query" in case:
        from oracle import qsa_select as Sel
        with _blas_limit(threads):
            loop(lambda: Sel.run_select_case(case))
        return n, busy, case["N"], (f"the full batch ({case['N']} query tokens), float64 "
                                    "oracle, numpy, one sequence at a time")
    if case.get("mode") == "mla_paged":
        from oracle import mla_kv_head as M
        sample = 2048
        caches = {k: spec.numpy() for k, spec in case["caches"].items()}
        args = (case["x"][:sample], case["w"], case["gamma"], case["alpha"], case["cos"][:sample],
                case["sin"][:sample], case["slot_mapping"][:sample], caches["k_cache"],
                caches["ckv_cache"], case["eps"], caches.get("ckv_scale"),
                case.get("ckv_dtype", "bf16"))
        with _blas_limit(threads):
            loop(lambda: M.mla_kv_head_paged(*args))
        return n, busy, sample, (f"the first {sample} tokens of the batch, float64 oracle "
                                 "(the projection is numpy's float64 matrix product)")
    if "raw_index_keys" in case:
        loop(lambda: oracle.run_qsa_case(case, nthreads=threads))
        return n, busy, case["N"] * case["L"], ("the full batch, C oracle, OpenMP over "
                                                "(sequence, block)")
    caches = {k: spec.numpy() for k, spec in case["caches"].items()}
    args = (case["kv"], case["gamma"], case["cos"], case["sin"])
    if case["mode"] == "paged":
        fn = lambda: oracle.paged_norm_rope_cache(                          # noqa: E731
            *args, case["slot_mapping"], caches["k_cache"], caches["ckv_cache"],
            caches.get("ckv_scale"), eps=case["eps"], nthreads=threads)
    elif case["mode"] == "paged_blk":
        fn = lambda: oracle.paged_blk_norm_rope_cache(                      # noqa: E731
            *args, case["block_index"], caches["k_cache"], caches["ckv_cache"],
            caches.get("ckv_scale"), eps=case["eps"], nthreads=threads)
    else:
        fn = lambda: oracle.norm_rope_cache(                                # noqa: E731
            *args, case["index"], caches["k_cache"], caches["ckv_cache"],
            caches.get("ckv_scale"), eps=case["eps"], nthreads=threads)
    loop(fn)
    _, tokens = algorithmic_bytes(case)
    return n, busy, tokens, "the full batch, C oracle, OpenMP over tokens"


class _blas_limit:
    """Limit numpy's BLAS threads inside the block (no-op if unavailable)."""

    def __init__(self, n):
        self.n, self.ctl = n, None

    def __enter__(self):
        try:
            from threadpoolctl import threadpool_limits
            self.ctl = threadpool_limits(limits=self.n, user_api="blas")
        except Exception:
            self.ctl = None
        return self

    def __exit__(self, *exc):
        if self.ctl is not None:
            self.ctl.restore_original_limits()
        return False


def cpu_baseline(case, seconds=8.0):
    """The oracle, as it is, on the host: one run of about `seconds` on one
    thread and one on every thread the oracle may use (OpenMP, or numpy's
    BLAS for the float64 oracles); value and cores are the all-threads run."""
    import oracle
    numpy_oracle = ("block_keys" in case and "query" in case) or case.get("mode") == "mla_paged"
    all_threads = _blas_threads() if numpy_oracle else oracle.max_threads()
    n1, b1, tok, what = _oracle_run(case, 1, seconds)
    na, ba, _, _ = _oracle_run(case, all_threads, seconds)
    return {"value": round(tok * na / ba, 1), "unit": "tokens/s", "cores": all_threads,
            "kind": "oracle",
            "single_thread_value": round(tok * n1 / b1, 1),
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{what}: {tok} tokens per run; {na} runs on {all_threads} threads "
                      f"({ba:.1f} s) and {n1} runs on 1 thread ({b1:.1f} s); input "
                      f"generation and cache allocation excluded"}


def _blas_threads() -> int:
    """Threads of numpy's BLAS (the float64 oracle's matrix product)."""
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(n[0])
    except Exception:
        pass
    return os.cpu_count() or 1


def read_traffic(workload):
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash(workload):
        return None
    return t.get("bytes_per_launch")


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find_csv(d, suffix):
    """The newest *suffix file under d (a directory reused by several runs
    keeps the older files)."""
    found = [os.path.join(root, f) for root, _, files in os.walk(d) for f in files
             if f.endswith(suffix)]
    if not found:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return max(found, key=os.path.getmtime)


def ingest_profile(args) -> int:
    """Summarise rocprofv3 output of this bench into profiles/:
    <kernel>_<workload>.md (kernel-trace stats, counters, commands) and
    traffic_<workload>.json (HBM bytes per launch, read back by the bench).

    Counters: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from two --pmc runs
    of `bench.py --calib-copy-mib 1024`; each is scaled by copy_bytes / value
    read on the 1 GiB device copy (the last 5 copyBuffer dispatches of the
    run), which turns the counter into bytes."""
    w = args.workload
    kname = KERNEL_NAME[kernel_family(w)]
    stats = [r for r in _csv_rows(_find_csv(args.trace_dir, "kernel_stats.csv"))
             if kname in r["Name"]]
    if not stats:
        raise SystemExit(f"{kname} not in the kernel-trace stats")
    st = stats[0]
    out = {"workload": w, "kernel": st["Name"], "source_hash": source_hash(w),
           "trace": {"calls": int(st["Calls"]), "avg_ns": float(st["AverageNs"]),
                     "min_ns": float(st["MinNs"]), "max_ns": float(st["MaxNs"])},
           "commands": args.command}
    # per-dispatch durations from the trace itself: percentiles of the kernel,
    # and the reference kernels of the same run (empty kernel per grid shape,
    # the same-bytes copy)
    import numpy as np
    trace = _csv_rows(_find_csv(args.trace_dir, "kernel_trace.csv"))

    def durations(pred):
        return np.array([int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in trace
                         if pred(r)], dtype=np.float64)

    d = durations(lambda r: r["Kernel_Name"] == st["Name"])
    if len(d):
        for p, v in zip((10, 50, 90), np.percentile(d, [10, 50, 90])):
            out["trace"][f"p{p}_ns"] = float(v)
    ctx = {}
    for r in trace:
        name = r["Kernel_Name"]
        if "empty_kernel" in name:
            key = (f"empty_kernel, {r['Grid_Size_X']} threads in workgroups of "
                   f"{r['Workgroup_Size_X']}")
        elif "copy_kernel" in name:
            key = f"copy_kernel, {r['Grid_Size_X']} threads"
        else:
            continue
        ctx.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out["reference_kernels"] = {
        key: {"calls": len(v), "avg_ns": round(float(np.mean(v)), 1),
              "p50_ns": float(np.percentile(v, 50))} for key, v in sorted(ctx.items())}
    copy_bytes = 1024 * 2 ** 20
    for counter, d in (("FETCH_SIZE", args.fetch_dir), ("WRITE_SIZE", args.write_dir)):
        rows = _csv_rows(_find_csv(d, "counter_collection.csv"))
        mine = [float(r["Counter_Value"]) for r in rows
                if kname in r["Kernel_Name"] and r["Counter_Name"] == counter]
        copies = [r for r in rows if "copyBuffer" in r["Kernel_Name"] and r["Counter_Name"] == counter]
        copies.sort(key=lambda r: int(r["Dispatch_Id"]))
        calib = [float(r["Counter_Value"]) for r in copies[-5:]]
        kib = sum(mine) / len(mine)
        cal = sum(calib) / len(calib)
        factor = copy_bytes / (cal * 1024)
        out[counter] = {"kib_per_dispatch": round(kib, 3), "dispatches": len(mine),
                        "copy_kib": round(cal, 3), "scale": round(factor, 5),
                        "bytes_per_dispatch": round(kib * 1024 * factor)}
        # the bench's reference kernels in the same run: the empty kernel per
        # grid shape (the fixed traffic of a launch) and the same-bytes copy
        ref = {}
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            if "empty_kernel" in r["Kernel_Name"]:
                key = (f"empty_kernel, {r['Grid_Size']} threads in workgroups of "
                       f"{r['Workgroup_Size']}")
            elif "copy_kernel" in r["Kernel_Name"]:
                key = f"copy_kernel, {r['Grid_Size']} threads"
            else:
                continue
            ref.setdefault(key, []).append(float(r["Counter_Value"]))
        for key, v in ref.items():
            out.setdefault("reference_kernel_traffic", {}).setdefault(key, {})[counter] = \
                round(sum(v) / len(v) * 1024 * factor)
    out["bytes_per_launch"] = out["FETCH_SIZE"]["bytes_per_dispatch"] + \
        out["WRITE_SIZE"]["bytes_per_dispatch"]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"traffic_{w}.json"), "w") as f:
        json.dump(out, f, indent=1)
    import gen
    alg, tokens = algorithmic_bytes(gen.make_config(w))
    avg_s = out["trace"]["avg_ns"] * 1e-9
    bench_line = open(args.bench_json).read().strip() if args.bench_json else None
    md = [f"# {kname} - {w}", "",
          f"Workload: {WORKLOAD_TEXT[w]}.", "",
          "Commands (from the repository root, on one MI355X):", ""]
    md += [f"    {c}" for c in args.command] + [""]
    md += ["## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
           "| kernel | calls | avg ns | min ns | max ns |", "|---|---|---|---|---|",
           f"| `{st['Name']}` | {st['Calls']} | {float(st['AverageNs']):.1f} | {st['MinNs']} | "
           f"{st['MaxNs']} |", ""]
    tr = out["trace"]
    if "p50_ns" in tr:
        md += [f"Per-dispatch duration percentiles (kernel trace): p10 {tr['p10_ns']:.0f} ns, "
               f"p50 {tr['p50_ns']:.0f} ns, p90 {tr['p90_ns']:.0f} ns.", ""]
    if out["reference_kernels"]:
        md += ["Reference kernels of the same run (bench context: empty kernel per grid "
               "shape = launch floor; plain copy of the same bytes = bandwidth ceiling):", "",
               "| kernel | calls | avg ns | p50 ns |", "|---|---|---|---|"]
        md += [f"| {key} | {v['calls']} | {v['avg_ns']} | {v['p50_ns']:.0f} |"
               for key, v in out["reference_kernels"].items()]
        md += [""]
    md += [
           f"Algorithmic bytes per launch: {alg} ({tokens} tokens) -> "
           f"{alg / avg_s / 1e9:.1f} GB/s at the average duration "
           f"({alg / avg_s / 8e12 * 100:.1f} % of 8 TB/s).", ""]
    flops = algorithmic_flops(gen.make_config(w))
    if flops:
        md += [f"Algorithmic flops per launch: {flops} (2 * T * 576 * He) -> "
               f"{flops / avg_s / 1e12:.1f} TFLOP/s at the average duration "
               f"({flops / avg_s / 1e12 / MFMA_BF16_PEAK_TFLOPS * 100:.1f} % of the "
               f"{MFMA_BF16_PEAK_TFLOPS:.0f} TFLOP/s bf16 dense peak).", ""]
    md += [
           "## HBM traffic (rocprofv3 --pmc, one counter per run)", "",
           "| counter | KiB per dispatch | on the 1 GiB copy | scale | bytes per dispatch |",
           "|---|---|---|---|---|"]
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        c = out[counter]
        md.append(f"| {counter} | {c['kib_per_dispatch']} | {c['copy_kib']} | {c['scale']} | "
                  f"{c['bytes_per_dispatch']} |")
    md += ["", f"Measured traffic per launch: {out['bytes_per_launch']} bytes "
               f"({out['bytes_per_launch'] / alg * 100:.1f} % of the algorithmic bytes); "
               f"{out['bytes_per_launch'] / avg_s / 1e9:.1f} GB/s at the average duration."]
    if out.get("reference_kernel_traffic"):
        md += ["", "The same counters on the bench's reference kernels (bytes per dispatch, "
                   "scaled alike):", "", "| kernel | FETCH_SIZE bytes | WRITE_SIZE bytes |",
               "|---|---|---|"]
        md += [f"| {key} | {v.get('FETCH_SIZE')} | {v.get('WRITE_SIZE')} |"
               for key, v in sorted(out["reference_kernel_traffic"].items())]
    md += [
           "", f"Kernel sources hash: {out['source_hash']}."]
    if bench_line:
        md += ["", "## bench.py line of the same run", "", "    " + bench_line]
    name = kname + ("_d576" if kname == "norm_rope_cache" else "")
    with open(os.path.join(ROOT, "profiles", f"{name}_{w}.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(md))
    return 0


def _gate(stream, ms=5.0):
    """Keep the GPU busy for about `ms` milliseconds on `stream` (a spin
    kernel), so that the launches enqueued behind it are all submitted before
    the first of them starts: the timed region then holds GPU work only."""
    import torch
    with torch.cuda.stream(stream):
        torch.cuda._sleep(int(ms * 2.0e6))


def _percentiles(xs, ps=(10, 50, 90)):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {f"p{p}": round(float(np.percentile(a, p)), 3) for p in ps}


def _time_graph(launches, stream):
    """Capture `launches` (callables, one launch each) into one HIP graph and
    time one replay with HIP events on `stream`: (elapsed ms, replay fn)."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for f in launches:
            f()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    _gate(stream)
    e0.record(stream)
    with torch.cuda.stream(stream):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1), g


def isolated_launch_times(launches, stream):
    """Per-launch durations (us): each launch bracketed by its own pair of
    timing events, behind a short spin kernel so that the launch and its end
    event are already queued when the start event is reached. Each figure is
    one launch's execution plus the event pair's own overhead, with the
    stream otherwise idle."""
    import torch
    pairs = []
    with torch.cuda.stream(stream):
        for f in launches:
            torch.cuda._sleep(100000)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            f()
            b.record(stream)
            pairs.append((a, b))
    torch.cuda.synchronize()
    d = [a.elapsed_time(b) * 1e3 for a, b in pairs]
    out = _percentiles(d)
    out["mean"] = round(sum(d) / len(d), 3)
    out["launches"] = len(d)
    return out


def kvrc_grid(case):
    """(workgroups, threads) of the norm-rope-cache launch for the workload's
    shape: Dv = 512 / Dk = 64 runs one row per one-wavefront workgroup up to
    2048 tokens and 2 rows per wavefront in 256-thread workgroups above;
    other shapes one row per wavefront in 256-thread workgroups."""
    T = case["B"] * case["S"]
    if case["Dv"] == 512 and case["Dk"] == 64:
        return (T, 64) if T <= 2048 else (-(-T // 8), 256)
    return -(-T // 4), 256


def context_measurements(case, bytes_per_launch, steps, stream, dev):
    """Reference points measured in the same harness (graph of `steps`
    launches, events on the launch stream): the launch floor of an empty
    kernel (one 64-thread workgroup, and the workload's grid where it is the
    norm-rope-cache kernel), and a plain device copy moving the same bytes as
    one launch (bytes/2 read, bytes/2 written) over buffers rotated past the
    Infinity Cache."""
    import torch
    import latent_attention_kv_amd as k
    out = {}
    ms, _ = _time_graph([lambda: k.kvrc_selftest_empty(1, 64)] * steps, stream)
    out["empty_kernel_1wg_us"] = round(ms * 1e3 / steps, 3)
    if kernel_family_of_case(case) == "kvrc":
        wg, th = kvrc_grid(case)
        ms, _ = _time_graph([lambda: k.kvrc_selftest_empty(wg, th)] * steps, stream)
        out["empty_kernel_same_grid_us"] = round(ms * 1e3 / steps, 3)
        out["same_grid"] = [wg, th]
    half = (bytes_per_launch // 2) // 16 * 16
    pairs = max(2, -(-512 * 2 ** 20 // (2 * half)))
    bufs = [(torch.empty(half, dtype=torch.uint8, device=dev).fill_(1),
             torch.empty(half, dtype=torch.uint8, device=dev)) for _ in range(pairs)]
    launches = [(lambda s=s, d=d: k.kvrc_selftest_copy(s, d)) for s, d in bufs]
    ms, _ = _time_graph([launches[i % pairs] for i in range(steps)], stream)
    us = ms * 1e3 / steps
    out["copy_same_bytes_us"] = round(us, 3)
    out["copy_same_bytes_gbps"] = round(2 * half / (us * 1e-6) / 1e9, 1)
    out["copy_bytes_read_and_written"] = 2 * half
    del bufs
    torch.cuda.empty_cache()
    return out


def kernel_family_of_case(case):
    if "block_keys" in case and "query" in case:
        return "sel"
    if case.get("mode") == "mla_paged":
        return "mla"
    if "raw_index_keys" in case:
        return "qsa"
    return "kvrc"


def cpu_model() -> str:
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for ln in out.splitlines():
            if ln.startswith("Model name:"):
                return ln.split(":", 1)[1].strip()
    except Exception:
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def read_profile_times(workload):
    """Per-dispatch durations of the kernel from the committed rocprofv3
    trace summary (only while the kernel sources are unchanged)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash(workload):
        return None
    tr = t.get("trace", {})
    out = {"avg_us": round(tr["avg_ns"] / 1e3, 3), "calls": tr.get("calls")}
    for p in ("p10", "p50", "p90"):
        if f"{p}_ns" in tr:
            out[f"{p}_us"] = round(tr[f"{p}_ns"] / 1e3, 3)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="prefill_paged", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--sets", type=int, default=0,
                    help="buffer sets rotated (0: enough to exceed 512 MB touched)")
    ap.add_argument("--timing", choices=["queued", "graph"], default="queued",
                    help="queued: the launches are enqueued behind a spin kernel long enough to "
                         "cover their submission, then run back to back; graph: a warm-up and "
                         "a timed HIP graph, replayed back to back")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="oracle time per CPU baseline run (one thread, then all threads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the per-step percentiles, launch floor and copy ceiling")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this size 5 times "
                         "(counter calibration under rocprofv3)")
    ap.add_argument("--ingest-profile", action="store_true",
                    help="summarise rocprofv3 output into profiles/ (no GPU needed)")
    ap.add_argument("--trace-dir")
    ap.add_argument("--fetch-dir")
    ap.add_argument("--write-dir")
    ap.add_argument("--bench-json")
    ap.add_argument("--command", action="append", default=[])
    args = ap.parse_args(argv)

    if args.ingest_profile:
        return ingest_profile(args)
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by sequence with no exchange; no multi-GPU run exists)",
              file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("bench.py: --steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch

    import gen
    import latent_attention_kv_amd as k

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    k.lib()
    dev = torch.device("cuda:0")
    case = gen.make_config(args.workload)
    bytes_per_launch, tokens = algorithmic_bytes(case)
    R = args.sets or max(2, min(64, -(-512 * 2 ** 20 // max(1, touched_bytes(case)))))
    sets = build_sets(case, R, dev)
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()
    # one eager launch per buffer set: loads the library and checks every
    # argument set once (setup, neither warm-up nor timed); it also gives the
    # host's cost of one launch call
    with torch.cuda.stream(stream):
        launch(case, sets[0])
        h0 = time.perf_counter()
        for s in sets:
            launch(case, s)
        host_us = (time.perf_counter() - h0) / R * 1e6
    stream.synchronize()

    def launch_fn(i):
        s = sets[i % R]
        return lambda: launch(case, s)

    W, K = args.warmup, args.steps
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    host_ahead = None
    if args.timing == "queued":
        # A spin kernel long enough for the host to enqueue every launch
        # (twice the measured host cost, at least 5 ms), then W warm-up and K
        # timed launches: the GPU runs them back to back, with nothing
        # between two launches but the dispatch of the next. The event after
        # the spin kernel tells whether the host finished enqueuing first.
        gate_ms = max(5.0, 2e-3 * (W + K) * host_us)
        _gate(stream, gate_ms)
        eg = torch.cuda.Event()
        eg.record(stream)
        with torch.cuda.stream(stream):
            for i in range(W):
                launch(case, sets[i % R])
            e0.record(stream)
            for i in range(W, W + K):
                launch(case, sets[i % R])
            e1.record(stream)
        host_ahead = not eg.query()
        torch.cuda.synchronize()
    else:
        # warm-up: W launches in one graph; timed: exactly K launches in one
        # graph, continuing the rotation; a spin kernel, then both graphs back
        # to back (the gap between the two graphs falls in the timed region)
        if W:
            gw = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gw, stream=stream):
                for i in range(W):
                    launch(case, sets[i % R])
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(W, W + K):
                launch(case, sets[i % R])
        torch.cuda.synchronize()
        _gate(stream)
        if W:
            with torch.cuda.stream(stream):
                gw.replay()
        e0.record(stream)
        with torch.cuda.stream(stream):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    secs = ms / 1e3
    kernel_us = ms * 1e3

    context = None
    if not args.no_context:
        n_iso = min(K, 200)
        context = {"isolated_launch_us": isolated_launch_times(
            [launch_fn(i) for i in range(W, W + n_iso)], stream)}
        context.update(context_measurements(case, bytes_per_launch, K, stream, dev))
    if args.calib_copy_mib:
        n = args.calib_copy_mib * 2 ** 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()

    achieved = bytes_per_launch / (kernel_us * 1e-6) / 1e9
    flops = algorithmic_flops(case)
    if flops:
        tflops = flops / (kernel_us * 1e-6) / 1e12
        roofline = {"bound": "mfma", "achieved": round(tflops, 1),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                    "traffic": read_traffic(args.workload),
                    "algorithmic_flops_per_launch": flops,
                    "algorithmic_bytes_per_launch": bytes_per_launch,
                    "hbm_gbps_at_algorithmic_bytes": round(achieved, 1),
                    "kernel_us": round(kernel_us, 3)}
    else:
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                    "traffic": read_traffic(args.workload),
                    "algorithmic_bytes_per_launch": bytes_per_launch,
                    "kernel_us": round(kernel_us, 3)}
    prof = read_profile_times(args.workload)
    roofline["rocprof_kernel_us"] = prof
    if prof:
        ach = (flops / 1e12 if flops else bytes_per_launch / 1e9) / (prof["avg_us"] * 1e-6)
        roofline["rocprof_frac"] = round(ach / (MFMA_BF16_PEAK_TFLOPS if flops
                                                 else HBM_PEAK_GBPS), 4)
    line = {
        "metric": METRIC,
        "value": round(tokens / secs, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if flops else "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {WORKLOAD_TEXT[args.workload]}",
                   "tokens_per_step": tokens, "io_dtype": "bf16",
                   "buffer_sets_rotated": R, "timing": args.timing,
                   "host_enqueued_ahead": host_ahead, "host_us_per_launch": round(host_us, 1),
                   "setup_launches": R + 1},
        "roofline": roofline,
    }
    if context is not None:
        line["context"] = context
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
