#!/usr/bin/env python3
"""Benchmark of the large-beam decode-attention hot path on one MI355X.

One step = one gr_decode_attn call over a whole batch: the shared-context
stage, the per-beam BeamPath stage and the log-sum-exp merge for every
(request, beam, head).  Inputs are seeded synthetic tensors with the
workloads' shapes, resident in HBM before timing starts; consecutive steps
rotate over enough copies of the inputs (more than twice the 256 MB
Infinity Cache) that every step reads them from HBM.

Prints ONE JSON line.  The headline workload is the Qwen3-0.6B attention
shape at 128 beams (B=8, ctx 1024, HBM-bound); the 900-beam workload
(MFMA-bound) is measured the same way and reported under "secondary".  The
per-beam state update of the same decode step (gr_beam_step: BeamKV append
+ BeamPath update, HBM-bound) is reported under "beam_step" at the 900- and
128-beam shapes.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from shared_prefix_beam_amd import inputs as I  # noqa: E402

METRIC = "GR decode-attn beam-rows/s + % bf16 MFMA peak (W=900), HBM GB/s (W=128)"
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
MALL_BYTES = 256 << 20
PRIMARY = 2                   # Qwen3-0.6B shape, W=128
SECONDARY = 4                 # Qwen3-0.6B shape, W=900
KERNEL_SOURCES = ["shared_prefix_beam_amd/csrc/gr_attn_kernels.hip",
                  "shared_prefix_beam_amd/csrc/gr_attn16.hip",
                  "shared_prefix_beam_amd/csrc/gr_attn_device.h",
                  "shared_prefix_beam_amd/csrc/gr_attn_internal.h",
                  "shared_prefix_beam_amd/csrc/gr_attn_api.cpp"]
STEP_SOURCES = ["shared_prefix_beam_amd/csrc/gr_beam_step.hip"]
STEP_CFGS = (4, 2)            # beam-step shapes reported (900 and 128 beams)
SELECT_SOURCES = ["shared_prefix_beam_amd/csrc/gr_beam_select.hip"]
SELECT_CFGS = (4, 2)          # beam-selection shapes reported (900 and 128 beams)
SELECT_KERNELS = ("select_rows", "select_request")
TRIE_CFGS = (4,)              # constrained-selection shape reported (900 beams, second step)
PAGE_SIZE = 16                # tokens per page of the paged-ContextKV measurement


def algorithmic(inp: I.Inputs):
    """(bytes, flops) the method must move / compute, each counted once.

    bytes: ContextKV K+V of every (request, KV head) once, q and out once,
    fp32 LSE, the BeamPath entries in use and every distinct BeamKV row a
    path references (K+V).  flops: 4*W*Hq*D*L per request for the shared
    stage (QK^T and PV); the beam stage and softmax are not counted.
    """
    wl = inp.wl
    U = I.unique_beam_rows(inp)
    nbytes = 0
    flops = 0
    for b in range(inp.B):
        Wb = int(inp.row_offset[b + 1] - inp.row_offset[b])
        L = int(inp.ctx_len[b])
        T = int(inp.beam_len[b])
        nbytes += 4 * L * wl.Hkv * wl.D + 4 * Wb * wl.Hq * wl.D + 4 * Wb * wl.Hq \
            + 4 * Wb * T + 4 * U[b] * wl.Hkv * wl.D
        flops += 4 * Wb * wl.Hq * wl.D * L
    return nbytes, flops


def algorithmic_step(st: I.StepInputs) -> int:
    """Bytes one beam step must move, each once: the new K and V rows read
    and written into their slots, the parent index, the parent's s path
    entries read and s+1 entries written, and per request the two lengths
    and two row offsets."""
    s = st.state
    row = s.wl.Hkv * s.wl.D * 2                        # bytes of one token's K (or V)
    nbytes = 0
    for b in range(s.B):
        w_new = int(st.row_offset_new[b + 1] - st.row_offset_new[b])
        t = int(s.beam_len[b])
        nbytes += w_new * (4 * row + 4 + 4 * t + 4 * (t + 1)) + 16
    return nbytes


def algorithmic_select(si: I.SelectInputs) -> int:
    """Bytes one beam selection must move, each once: every logit and old
    score read, the two row-offset arrays read, and (score, parent, token)
    written per kept beam."""
    R_old, V = si.logits.shape
    B = si.row_offset_old.size - 1
    R_new = int(si.row_offset_new[-1])
    return 4 * R_old * V + 4 * R_old + 8 * (B + 1) + 12 * R_new


def algorithmic_trie(ti: I.TrieSelectInputs) -> int:
    """Bytes one constrained selection must move, each once: per beam its
    node id, the node's two CSR offsets and its score; per legal edge its
    label and the logit it selects; the row offsets; and per kept beam the
    score, parent, token and node written, with the chosen edge's label and
    child read."""
    si, tr = ti.sel, ti.trie
    fan = np.diff(tr.node_ptr)
    live = ti.node_old >= 0
    n_edges = int(fan[ti.node_old[live]].sum())
    R_old = si.logits.shape[0]
    B = si.row_offset_old.size - 1
    R_new = int(si.row_offset_new[-1])
    return 4 * R_old + 4 * R_old + 8 * int(live.sum()) + 8 * n_edges + 8 * (B + 1) + 24 * R_new


def kernel_hash(sources=None) -> str:
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES if sources is None else sources):
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, kernel: str = "fused_decode_attn", sources=None):
    """HBM traffic per launch from a committed rocprofv3 --pmc summary, if it
    was taken from the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_sha") != kernel_hash(sources):
        return None
    return rec.get("bytes_per_launch")


# rocprofv3 runs behind the committed summaries in profiles/ (run from the
# repository root on the GPU machine; {d} is the output folder)
PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d {d}/trace_{w} -o trace "
             "-- python3 bench.py --only {w} --steps 100 --warmup 10",
    "fetch": "timeout -s KILL 60 rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/fetch_{w} "
             "-o fetch -- python3 bench.py --only {w} --steps 5 --warmup 1",
    "write": "timeout -s KILL 60 rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/write_{w} "
             "-o write -- python3 bench.py --only {w} --steps 5 --warmup 1",
    "copy_fetch": "timeout -s KILL 60 rocprofv3 --pmc FETCH_SIZE --output-format csv "
                  "-d {d}/copy_fetch -o copy_fetch -- python3 bench.py --copy-calibration",
    "copy_write": "timeout -s KILL 60 rocprofv3 --pmc WRITE_SIZE --output-format csv "
                  "-d {d}/copy_write -o copy_write -- python3 bench.py --copy-calibration",
}
COPY_BYTES = 256 << 20


def _csv_rows(folder: str, suffix: str):
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {folder}")
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    return rows


def _counter_per_dispatch(folder: str, kernel_substr: str, counter: str):
    """Mean counter value (KiB) over the dispatches of one kernel."""
    vals = [float(r["Counter_Value"]) for r in _csv_rows(folder, "counter_collection.csv")
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not vals:
        raise ValueError(f"no {counter} rows for {kernel_substr} in {folder}")
    return float(np.mean(vals)), len(vals)


def _copy_factor(folder: str, counter: str):
    """Bytes per counted KiB, from the 256 MiB copies of --copy-calibration."""
    vals = [float(r["Counter_Value"]) for r in _csv_rows(folder, "counter_collection.csv")
            if "copyBuffer" in r["Kernel_Name"] and r["Counter_Name"] == counter]
    big = sorted(vals)[-10:]
    kib = float(np.mean(big))
    return COPY_BYTES / (kib * 1024.0), kib


def write_profile_summaries(d: str):
    """Turn the rocprofv3 outputs under `d` (made by PROFILE_COMMANDS) into the
    text summaries and the per-launch traffic records kept in profiles/."""
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    f_fetch, copy_fetch_kib = _copy_factor(os.path.join(d, "copy_fetch"), "FETCH_SIZE")
    f_write, copy_write_kib = _copy_factor(os.path.join(d, "copy_write"), "WRITE_SIZE")
    sha = kernel_hash()
    for which, cfg, page in (("primary", PRIMARY, None), ("secondary", SECONDARY, None),
                             ("cfg1", 1, None), ("cfg3", 3, None), ("cfg5", 5, None),
                             ("paged2", 2, PAGE_SIZE), ("paged4", 4, PAGE_SIZE)):
        if not os.path.isdir(os.path.join(d, f"trace_{which}")):
            continue                                # not profiled in this folder
        wl = I.WORKLOADS[cfg]
        stats = [r for r in _csv_rows(os.path.join(d, f"trace_{which}"), "kernel_stats.csv")]
        fetch_kib, n_f = _counter_per_dispatch(os.path.join(d, f"fetch_{which}"),
                                              "fused_decode_attn", "FETCH_SIZE")
        write_kib, n_w = _counter_per_dispatch(os.path.join(d, f"write_{which}"),
                                              "fused_decode_attn", "WRITE_SIZE")
        traffic = fetch_kib * 1024 * f_fetch + write_kib * 1024 * f_write
        inp = I.generate(wl)
        nbytes, flops = algorithmic(inp)
        tag = wl.name if page is None else f"paged{page}_{wl.name}"
        title = wl.name if page is None else f"{wl.name}, ContextKV in pages of {page} tokens"
        if page is not None:
            # plus each request's page table, read once
            nbytes += 4 * inp.B * max(-(-inp.ctx_cap // page), 1)
        kern = [r for r in stats if "fused_decode_attn" in r["Name"]]
        kname = kern[0]["Name"] if kern else "fused_decode_attn"
        lines = [f"# fused decode attention on {title}", "", f"kernel: {kname}", "",
                 "kernel trace (rocprofv3 --kernel-trace --stats), command from the repository root:",
                 "    " + PROFILE_COMMANDS["trace"].format(d="gpurun_out/prof", w=which), "",
                 f"{'kernel':60s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
        for r in stats:
            lines.append(f"{r['Name'][:60]:60s} {int(r['Calls']):6d} "
                         f"{float(r['AverageNs']) / 1e3:9.2f} {float(r['MinNs']) / 1e3:9.2f} "
                         f"{float(r['MaxNs']) / 1e3:9.2f}")
        avg_us = float(kern[0]["AverageNs"]) / 1e3 if kern else float("nan")
        lines += ["", "HBM counters, one pass each:",
                  "    " + PROFILE_COMMANDS["fetch"].format(d="gpurun_out/prof", w=which),
                  "    " + PROFILE_COMMANDS["write"].format(d="gpurun_out/prof", w=which),
                  "    " + PROFILE_COMMANDS["copy_fetch"].format(d="gpurun_out/prof"),
                  "    " + PROFILE_COMMANDS["copy_write"].format(d="gpurun_out/prof"), "",
                  f"FETCH_SIZE per dispatch   {fetch_kib:12.1f} KiB  (mean of {n_f})",
                  f"WRITE_SIZE per dispatch   {write_kib:12.1f} KiB  (mean of {n_w})",
                  f"copy of 256 MiB reads     FETCH_SIZE {copy_fetch_kib:.1f} KiB -> "
                  f"{f_fetch:.3f} bytes per counted KiB/1024",
                  f"copy of 256 MiB writes    WRITE_SIZE {copy_write_kib:.1f} KiB -> "
                  f"{f_write:.3f} bytes per counted KiB/1024",
                  f"HBM traffic per launch    {traffic / 1e6:12.3f} MB",
                  f"algorithmic bytes         {nbytes / 1e6:12.3f} MB  "
                  f"(traffic / algorithmic = {traffic / nbytes:.3f})",
                  f"algorithmic flops         {flops / 1e9:12.3f} GFLOP",
                  f"average launch            {avg_us:12.2f} us -> "
                  f"{nbytes / avg_us / 1e3:.1f} GB/s, {flops / avg_us / 1e6:.1f} TFLOP/s",
                  f"kernel sources sha256[:16] {sha}"]
        name = f"fused_decode_attn_{tag}"
        open(os.path.join(out_dir, name + ".txt"), "w").write("\n".join(lines) + "\n")
        json.dump({"kernel": kname, "workload": tag, "kernel_sha": sha,
                   "bytes_per_launch": traffic, "fetch_kib": fetch_kib, "write_kib": write_kib,
                   "fetch_factor": f_fetch, "write_factor": f_write, "avg_launch_us": avg_us},
                  open(os.path.join(out_dir, f"traffic_{name}.json"), "w"), indent=1)
        print(f"wrote profiles/{name}.txt", flush=True)
    write_step_profile(d, f_fetch, f_write, copy_fetch_kib, copy_write_kib)
    write_step_profile(d, f_fetch, f_write, copy_fetch_kib, copy_write_kib, w="beam_step2")
    write_select_profile(d, f_fetch, f_write)
    write_select_profile(d, f_fetch, f_write, w="select2")
    write_select_profile(d, f_fetch, f_write, w="trie")


def write_step_profile(d, f_fetch, f_write, copy_fetch_kib, copy_write_kib, w="beam_step"):
    """The same summary for the beam-step kernel (profiled with --only beam_step for the
    900-beam shape, --only beam_step2 for the 128-beam one)."""
    if not os.path.isdir(os.path.join(d, f"trace_{w}")):
        return
    cfg = STEP_CFGS[1] if w == "beam_step2" else STEP_CFGS[0]
    st = I.step_workload(cfg)
    name_wl = I.STEP_WORKLOADS[cfg]["name"]
    nbytes = algorithmic_step(st)
    stats = _csv_rows(os.path.join(d, f"trace_{w}"), "kernel_stats.csv")
    fetch_kib, n_f = _counter_per_dispatch(os.path.join(d, f"fetch_{w}"), "beam_step",
                                          "FETCH_SIZE")
    write_kib, n_w = _counter_per_dispatch(os.path.join(d, f"write_{w}"), "beam_step",
                                          "WRITE_SIZE")
    traffic = fetch_kib * 1024 * f_fetch + write_kib * 1024 * f_write
    kern = [r for r in stats if "beam_step" in r["Name"]]
    avg_us = float(kern[0]["AverageNs"]) / 1e3 if kern else float("nan")
    sha = kernel_hash(STEP_SOURCES)
    lines = [f"# beam_step on {name_wl}", "",
             "kernel trace (rocprofv3 --kernel-trace --stats), command from the repository root:",
             "    " + PROFILE_COMMANDS["trace"].format(d="gpurun_out/prof", w=w), "",
             f"{'kernel':60s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
    for r in stats:
        lines.append(f"{r['Name'][:60]:60s} {int(r['Calls']):6d} "
                     f"{float(r['AverageNs']) / 1e3:9.2f} {float(r['MinNs']) / 1e3:9.2f} "
                     f"{float(r['MaxNs']) / 1e3:9.2f}")
    lines += ["", "HBM counters, one pass each:",
              "    " + PROFILE_COMMANDS["fetch"].format(d="gpurun_out/prof", w=w),
              "    " + PROFILE_COMMANDS["write"].format(d="gpurun_out/prof", w=w),
              "    (copy calibration as in the attention summaries)", "",
              f"FETCH_SIZE per dispatch   {fetch_kib:12.1f} KiB  (mean of {n_f})",
              f"WRITE_SIZE per dispatch   {write_kib:12.1f} KiB  (mean of {n_w})",
              f"copy factors              fetch {f_fetch:.3f}, write {f_write:.3f}",
              f"HBM traffic per launch    {traffic / 1e6:12.3f} MB",
              f"algorithmic bytes         {nbytes / 1e6:12.3f} MB  "
              f"(traffic / algorithmic = {traffic / nbytes:.3f})",
              f"average launch            {avg_us:12.2f} us -> {nbytes / avg_us / 1e3:.1f} GB/s",
              f"kernel sources sha256[:16] {sha}"]
    name = f"beam_step_{name_wl}"
    out_dir = os.path.join(ROOT, "profiles")
    open(os.path.join(out_dir, name + ".txt"), "w").write("\n".join(lines) + "\n")
    json.dump({"kernel": "beam_step", "workload": name_wl, "kernel_sha": sha,
               "bytes_per_launch": traffic, "fetch_kib": fetch_kib, "write_kib": write_kib,
               "fetch_factor": f_fetch, "write_factor": f_write, "avg_launch_us": avg_us},
              open(os.path.join(out_dir, f"traffic_{name}.json"), "w"), indent=1)
    print(f"wrote profiles/{name}.txt", flush=True)


def write_select_profile(d, f_fetch, f_write, w="select"):
    """Summary of the two beam-selection kernels (profiled with --only select
    for the 900-beam shape, --only select2 for the 128-beam one, or --only trie
    for the constrained call): per-kernel averages and counters, summed per
    call."""
    if not os.path.isdir(os.path.join(d, f"trace_{w}")):
        return
    if w == "trie":
        ti = I.trie_workload(TRIE_CFGS[0])
        name_wl = I.TRIE_WORKLOADS[TRIE_CFGS[0]]["name"]
        nbytes = algorithmic_trie(ti)
        title, kname = "constrained beam selection", "beam_select_trie"
    else:
        cfg = SELECT_CFGS[1] if w == "select2" else SELECT_CFGS[0]
        name_wl = I.SELECT_WORKLOADS[cfg]["name"]
        nbytes = algorithmic_select(I.select_workload(cfg))
        title, kname = "beam selection", "beam_select"
    stats = _csv_rows(os.path.join(d, f"trace_{w}"), "kernel_stats.csv")
    sha = kernel_hash(SELECT_SOURCES)
    lines = [f"# {title} (select_rows + select_request) on {name_wl}", "",
             "kernel trace (rocprofv3 --kernel-trace --stats), command from the repository root:",
             "    " + PROFILE_COMMANDS["trace"].format(d="gpurun_out/prof", w=w), "",
             f"{'kernel':60s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
    for r in stats:
        lines.append(f"{r['Name'][:60]:60s} {int(r['Calls']):6d} "
                     f"{float(r['AverageNs']) / 1e3:9.2f} {float(r['MinNs']) / 1e3:9.2f} "
                     f"{float(r['MaxNs']) / 1e3:9.2f}")
    lines += ["", "HBM counters, one pass each:",
              "    " + PROFILE_COMMANDS["fetch"].format(d="gpurun_out/prof", w=w),
              "    " + PROFILE_COMMANDS["write"].format(d="gpurun_out/prof", w=w),
              "    (copy calibration as in the attention summaries)", ""]
    avg_us = 0.0
    traffic = 0.0
    per = {}
    for k in SELECT_KERNELS:
        kern = [r for r in stats if k in r["Name"]]
        us = float(kern[0]["AverageNs"]) / 1e3 if kern else float("nan")
        fk, n_f = _counter_per_dispatch(os.path.join(d, f"fetch_{w}"), k, "FETCH_SIZE")
        wk, n_w = _counter_per_dispatch(os.path.join(d, f"write_{w}"), k, "WRITE_SIZE")
        t = fk * 1024 * f_fetch + wk * 1024 * f_write
        per[k] = {"avg_launch_us": us, "fetch_kib": fk, "write_kib": wk, "bytes_per_launch": t}
        avg_us += us
        traffic += t
        lines.append(f"{k:16s} avg {us:9.2f} us  FETCH_SIZE {fk:10.1f} KiB  WRITE_SIZE "
                     f"{wk:10.1f} KiB  (means of {n_f}, {n_w})  -> {t / 1e6:8.3f} MB")
    lines += [f"copy factors              fetch {f_fetch:.3f}, write {f_write:.3f}",
              f"HBM traffic per call      {traffic / 1e6:12.3f} MB",
              f"algorithmic bytes         {nbytes / 1e6:12.3f} MB  "
              f"(traffic / algorithmic = {traffic / nbytes:.3f})",
              f"both kernels, per call    {avg_us:12.2f} us -> {nbytes / avg_us / 1e3:.1f} GB/s",
              f"kernel sources sha256[:16] {sha}"]
    name = f"{kname}_{name_wl}"
    out_dir = os.path.join(ROOT, "profiles")
    open(os.path.join(out_dir, name + ".txt"), "w").write("\n".join(lines) + "\n")
    json.dump({"kernel": kname, "workload": name_wl, "kernel_sha": sha,
               "bytes_per_launch": traffic, "per_kernel": per, "fetch_factor": f_fetch,
               "write_factor": f_write, "avg_launch_us": avg_us},
              open(os.path.join(out_dir, f"traffic_{name}.json"), "w"), indent=1)
    print(f"wrote profiles/{name}.txt", flush=True)


def spot_rows(inp: I.Inputs):
    """Rows checked against the oracle after timing: the first, middle and
    last row of every request that has rows."""
    rows = set()
    for b in range(inp.B):
        r0, r1 = int(inp.row_offset[b]), int(inp.row_offset[b + 1])
        if r1 > r0:
            rows.update((r0, (r0 + r1) // 2, r1 - 1))
    return sorted(rows)


def measure(cfg: int, steps: int, warmup: int, page_size=None, reps: int = 5,
            latency_calls: int = 20, settle=None):
    """Time gr_decode_attn on workload `cfg` (gr_decode_attn_paged with the
    context scattered over pages of `page_size` tokens when it is given).

    The timed region is `steps` back-to-back calls between two HIP events on
    the launch stream (rep 0: ms_per_step and the launch time of the bench
    line); `reps`-1 more such regions give the median and minimum.  Then
    `latency_calls` single calls, each after a 512 MB write that evicts the
    caches, with an event pair each, give the cold per-call latency.
    `settle`, when given, runs right before the warm-up steps (other GPU
    work that brings the clocks up after the host-side set-up)."""
    import torch
    from shared_prefix_beam_amd import gr_attn

    inp = I.generate(I.WORKLOADS[cfg])
    nbytes, flops = algorithmic(inp)
    base = I.to_torch(inp)
    if page_size:
        pg = I.to_paged(inp, page_size, seed=cfg)
        base["ctx_k"] = torch.from_numpy(pg.k_pages.view(np.int16)).view(torch.bfloat16).cuda()
        base["ctx_v"] = torch.from_numpy(pg.v_pages.view(np.int16)).view(torch.bfloat16).cuda()
        base["page_table"] = torch.from_numpy(pg.page_table.astype(np.int32)).cuda()
    footprint = sum(t.numel() * t.element_size() for t in base.values()) \
        + base["q"].numel() * 2 + base["q"].shape[0] * base["q"].shape[1] * 4
    # enough copies that each step reads HBM, at most 64 (a workload this
    # small is bound by launch latency, not by where its bytes come from)
    n_sets = min(64, max(2, int(np.ceil(2 * MALL_BYTES / footprint)) + 1))
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(n_sets - 1)]
    outs = [(torch.empty_like(s["q"]),
             torch.empty(s["q"].shape[:2], dtype=torch.float32, device="cuda")) for s in sets]
    W_max = int(max(inp.wl.W))
    stream = torch.cuda.current_stream()

    # one workspace (zeroed once) serves every call: the calls run in order
    # on one stream, and each leaves the split counters at zero
    dims = gr_attn.Dims(B=inp.B, R=inp.R, Hq=inp.wl.Hq, Hkv=inp.wl.Hkv, D=inp.wl.D,
                        W_max=W_max, T_cap=inp.T_cap, reserved=0, ctx_cap=inp.ctx_cap,
                        beam_cap=inp.beam_cap, scale=0.0, flags=0)
    workspace = gr_attn.attach_workspace(dims, None, "cuda")
    ws_bytes = int(dims.workspace_bytes)
    plan = gr_attn.plan(dims)

    # one front-end call per input copy validates shapes; the timed loop then
    # calls the C entry point directly with the same arguments
    if page_size:
        for s, (o, l) in zip(sets, outs):
            gr_attn.decode_attn_paged(s["q"], s["ctx_k"], s["ctx_v"], s["page_table"], page_size,
                                      s["ctx_len"], s["beam_k"], s["beam_v"], s["beam_path"],
                                      s["beam_len"], s["row_offset"], W_max=W_max,
                                      ctx_cap=inp.ctx_cap, out=o, lse=l, stream=stream,
                                      workspace=workspace)
        ctxs = [gr_attn.PagedCtx(k_pages=s["ctx_k"].data_ptr(), v_pages=s["ctx_v"].data_ptr(),
                                 page_table=s["page_table"].data_ptr(), page_size=page_size,
                                 pages_per_req=s["page_table"].shape[1],
                                 n_pages=s["ctx_k"].shape[0]) for s in sets]
        args = [tuple(t.data_ptr() for t in (s["row_offset"], s["q"], s["ctx_len"], s["beam_k"],
                                             s["beam_v"], s["beam_path"], s["beam_len"], o, l))
                for s, (o, l) in zip(sets, outs)]
    else:
        for s, (o, l) in zip(sets, outs):
            gr_attn.decode_attn(s["q"], s["ctx_k"], s["ctx_v"], s["ctx_len"], s["beam_k"],
                                s["beam_v"], s["beam_path"], s["beam_len"], s["row_offset"],
                                W_max=W_max, out=o, lse=l, stream=stream, workspace=workspace)
        args = [tuple(t.data_ptr() for t in (s["row_offset"], s["q"], s["ctx_k"], s["ctx_v"],
                                             s["ctx_len"], s["beam_k"], s["beam_v"],
                                             s["beam_path"], s["beam_len"], o, l))
                for s, (o, l) in zip(sets, outs)]
    handle = stream.cuda_stream

    def step(i):
        if page_size:
            st = gr_attn.gr_decode_attn_paged(dims, ctxs[i % n_sets], *args[i % n_sets], handle)
        else:
            st = gr_attn.gr_decode_attn(dims, *args[i % n_sets], handle)
        if st != gr_attn.GR_OK:
            raise gr_attn.GrAttnError(st, "gr_decode_attn")

    if settle is not None:
        settle()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: K back-to-back steps (one launch each), bracketed by
    # events recorded on the launch stream; the average launch duration is
    # their elapsed time / K, so the rate and the kernel duration come from
    # the same run.  No per-launch events, so the host never starves the GPU.
    launch = []
    ms_per_step = None
    for rep in range(max(1, reps)):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(steps):
            step(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        if rep == 0:
            ms_per_step = wall * 1e3 / steps
        launch.append(ev0.elapsed_time(ev1) / steps)

    # cold per-call latency: a 512 MB write between calls evicts L2 and MALL
    flush = torch.empty(512 << 20 if latency_calls else 1, dtype=torch.uint8, device="cuda")
    lat = []
    for i in range(latency_calls):
        flush.fill_(i & 255)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        lat.append(e0.elapsed_time(e1))
    del flush

    # spot check of a few rows against the oracle (not timed)
    from oracle import oracle as O
    rows = spot_rows(inp)
    out, lse = outs[0]
    step(0)
    torch.cuda.synchronize()
    ref_o, ref_l = O.decode_attn_inputs(inp, rows=rows)
    got_o = out.float().cpu().numpy()[rows]
    spot = float(np.abs(got_o - ref_o).max())
    fin = np.isfinite(ref_l)
    got_l = lse.cpu().numpy()[rows]
    spot_lse = float(np.abs(got_l[fin] - ref_l[fin]).max()) if fin.any() else 0.0

    srt = sorted(launch)
    return dict(inp=inp, nbytes=nbytes, flops=flops, ms_per_step=ms_per_step,
                launch_ms=launch[0], launch_median_ms=srt[len(srt) // 2], launch_min_ms=srt[0],
                launch_reps_ms=launch, latency_ms=sorted(lat)[len(lat) // 2] if lat else None,
                n_sets=n_sets, spot_abs=spot, spot_lse=spot_lse, spot_rows=len(rows),
                workspace_bytes=ws_bytes, plan=plan)


RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)   # flop per byte


def kernel_of(plan: dict) -> str:
    """The fused kernel a plan launches."""
    return "fused_decode_attn16" if plan["row16"] else "fused_decode_attn"


def config_entry(cfg: int, r) -> dict:
    """One workload's numbers: rates at the median launch time of the
    repetitions, both roofline fractions and which one bounds it."""
    inp = r["inp"]
    t = r["launch_median_ms"] * 1e-3
    gbs = r["nbytes"] / t / 1e9
    tf = r["flops"] / t / 1e12
    ai = r["flops"] / r["nbytes"]
    return {"config": cfg, "workload": inp.wl.name, "rows": inp.R, "heads": inp.wl.Hq,
            "launch_us": r["launch_ms"] * 1e3, "launch_us_median": r["launch_median_ms"] * 1e3,
            "launch_us_min": r["launch_min_ms"] * 1e3,
            "launch_us_reps": [round(x * 1e3, 3) for x in r["launch_reps_ms"]],
            "latency_us_cold": r["latency_ms"] * 1e3 if r["latency_ms"] is not None else None,
            "beam_rows_per_s": inp.R / t, "hbm_GBps": gbs, "hbm_frac": gbs / PEAK_HBM_GBS,
            "TFLOPs": tf, "mfma_frac": tf / PEAK_BF16_TFLOPS,
            "bound": "hbm" if ai < RIDGE else "mfma", "flop_per_byte": ai,
            "algorithmic_bytes": r["nbytes"], "algorithmic_flops": r["flops"],
            "kernel": kernel_of(r["plan"]), "plan": r["plan"],
            "workspace_bytes": r["workspace_bytes"], "traffic": recorded_traffic(inp.wl.name),
            "spot_check": {"rows": r["spot_rows"], "max_abs": r["spot_abs"],
                           "lse_abs": r["spot_lse"]}}


def measure_step(cfg: int, steps: int, warmup: int):
    """Time gr_beam_step on the step workload `cfg` the way `measure` times
    the attention: rotating input sets, direct C calls, one event pair per
    region of `steps` launches; five regions, their median reported (the kernel
    is about as short as one call's host-side cost, so a region in which the
    host falls behind measures the host)."""
    import torch
    from shared_prefix_beam_amd import gr_attn

    st = I.step_workload(cfg)
    s = st.state
    nbytes = algorithmic_step(st)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()

    base = dict(ro_old=i32(s.row_offset), ro_new=i32(st.row_offset_new), parent=i32(st.parent),
                path_old=i32(s.beam_path), len_old=i32(s.beam_len), new_k=bf(st.new_k),
                new_v=bf(st.new_v), path_new=i32(np.zeros((st.R_new, s.T_cap), np.int32)),
                len_new=i32(np.zeros(s.B, np.int32)), beam_k=bf(s.beam_k), beam_v=bf(s.beam_v))
    n_sets = max(2, int(np.ceil(2 * MALL_BYTES / nbytes)) + 1)
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(n_sets - 1)]
    stream = torch.cuda.current_stream()
    for t in sets:   # the front end validates every set once
        gr_attn.beam_step(t["ro_old"], t["ro_new"], t["parent"], t["path_old"], t["len_old"],
                          t["new_k"], t["new_v"], t["path_new"], t["len_new"], t["beam_k"],
                          t["beam_v"], s.W_cap, stream=stream)
    dims = gr_attn.StepDims(B=s.B, R_old=s.R, R_new=st.R_new, Hkv=s.wl.Hkv, D=s.wl.D,
                            T_cap=s.T_cap, W_cap=s.W_cap, reserved=0, beam_cap=s.beam_cap)
    order = ("ro_old", "ro_new", "parent", "path_old", "len_old", "new_k", "new_v", "path_new",
             "len_new", "beam_k", "beam_v")
    args = [tuple(t[k].data_ptr() for k in order) + (None,) for t in sets]
    handle = stream.cuda_stream

    def step(i):
        rc = gr_attn.gr_beam_step(dims, *args[i % n_sets], handle)
        if rc != gr_attn.GR_OK:
            raise gr_attn.GrAttnError(rc, "gr_beam_step")

    for i in range(warmup):
        step(i)
    reps = []
    for _ in range(5):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(steps):
            step(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        reps.append(ev0.elapsed_time(ev1) / steps)
    launch_ms = sorted(reps)[len(reps) // 2]
    # bit-exact spot check of the first set against the oracle (not timed)
    from oracle import oracle as O
    ref_path, ref_len, ref_k, ref_v, _ = O.beam_step(
        s.row_offset, st.row_offset_new, st.parent, s.beam_path, s.beam_len, st.new_k,
        st.new_v, np.zeros((st.R_new, s.T_cap), np.int32), s.beam_k, s.beam_v, s.W_cap)
    ok = (np.array_equal(base["path_new"].cpu().numpy(), ref_path)
          and np.array_equal(base["len_new"].cpu().numpy(), ref_len)
          and np.array_equal(base["beam_k"].view(torch.int16).cpu().numpy().view(np.uint16),
                             ref_k)
          and np.array_equal(base["beam_v"].view(torch.int16).cpu().numpy().view(np.uint16),
                             ref_v))
    return dict(st=st, name=I.STEP_WORKLOADS[cfg]["name"], nbytes=nbytes, launch_ms=launch_ms,
                reps_ms=reps, n_sets=n_sets, bit_exact=bool(ok))


def measure_select(cfg: int, steps: int, warmup: int, trie: bool = False):
    """Time gr_beam_select (gr_beam_select_trie with `trie`) on the selection
    workload `cfg` (both launches of one call between one event pair),
    rotating input sets like `measure`."""
    import torch
    from shared_prefix_beam_amd import gr_attn

    ti = I.trie_workload(cfg) if trie else None
    si = ti.sel if trie else I.select_workload(cfg)
    nbytes = algorithmic_trie(ti) if trie else algorithmic_select(si)
    R_old, V = si.logits.shape
    B = si.row_offset_old.size - 1
    R_new = int(si.row_offset_new[-1])
    K_max = int(np.diff(si.row_offset_new).max())
    dev = "cuda"
    base = dict(ro_old=torch.from_numpy(si.row_offset_old).to(dev),
                ro_new=torch.from_numpy(si.row_offset_new).to(dev),
                score_old=torch.from_numpy(si.score_old).to(dev),
                logits=torch.from_numpy(np.ascontiguousarray(si.logits)).to(dev))
    if trie:
        def i32(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
        base["node_old"] = i32(ti.node_old)
        t_trie = dict(node_ptr=i32(ti.trie.node_ptr), edge_tok=i32(ti.trie.edge_tok),
                      edge_child=i32(ti.trie.edge_child))
        # the largest fanout among this step's nodes (a catalog knows it per
        # level); it sizes the row launch
        fan = int(np.diff(ti.trie.node_ptr)[ti.node_old[ti.node_old >= 0]].max())
    # the logits dominate the bytes the sets occupy; rotate past the MALL
    set_bytes = 4 * R_old * V
    n_sets = max(2, int(np.ceil(2 * MALL_BYTES / set_bytes)) + 1)
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(n_sets - 1)]
    score_new = torch.empty(R_new, dtype=torch.float32, device=dev)
    parent = torch.empty(R_new, dtype=torch.int32, device=dev)
    token = torch.empty(R_new, dtype=torch.int32, device=dev)
    node_new = torch.empty(R_new, dtype=torch.int32, device=dev)
    dims = gr_attn.SelectDims(B=B, R_old=R_old, R_new=R_new, V=V, K_max=K_max, reserved=0)
    ws_bytes = gr_attn.gr_beam_select_workspace_bytes(dims)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    for t in sets:   # the front end validates every set once
        if trie:
            gr_attn.beam_select_trie(t["ro_old"], t["ro_new"], t["score_old"], t["logits"],
                                     t["node_old"], t_trie["node_ptr"], t_trie["edge_tok"],
                                     t_trie["edge_child"], K_max, fan, score_new=score_new,
                                     parent=parent, token=token, node_new=node_new,
                                     workspace=ws, stream=stream)
        else:
            gr_attn.beam_select(t["ro_old"], t["ro_new"], t["score_old"], t["logits"], K_max,
                                score_new=score_new, parent=parent, token=token, workspace=ws,
                                stream=stream)
    handle = stream.cuda_stream
    if trie:
        desc = gr_attn.SidTrie(node_ptr=t_trie["node_ptr"].data_ptr(),
                               edge_tok=t_trie["edge_tok"].data_ptr(),
                               edge_child=t_trie["edge_child"].data_ptr(),
                               n_nodes=ti.trie.n_nodes, n_edges=ti.trie.n_edges,
                               max_fanout=fan, reserved=0)
        args = [tuple(t[k].data_ptr() for k in ("ro_old", "ro_new", "score_old", "logits",
                                                 "node_old")) for t in sets]
        outs = (score_new.data_ptr(), parent.data_ptr(), token.data_ptr(), node_new.data_ptr(),
                ws.data_ptr(), ws_bytes)

        def call(i):
            rc = gr_attn.gr_beam_select_trie(dims, desc, *args[i % n_sets], *outs, handle)
            if rc != gr_attn.GR_OK:
                raise gr_attn.GrAttnError(rc, "gr_beam_select_trie")
    else:
        args = [tuple(t[k].data_ptr() for k in ("ro_old", "ro_new", "score_old", "logits"))
                for t in sets]
        outs = (score_new.data_ptr(), parent.data_ptr(), token.data_ptr(), ws.data_ptr(),
                ws_bytes)

        def call(i):
            rc = gr_attn.gr_beam_select(dims, *args[i % n_sets], *outs, handle)
            if rc != gr_attn.GR_OK:
                raise gr_attn.GrAttnError(rc, "gr_beam_select")

    for i in range(warmup):
        call(i)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(steps):
        call(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    launch_ms = ev0.elapsed_time(ev1) / steps
    # spot check against the oracle (not timed): the last call used set
    # (steps - 1) % n_sets, identical to the first
    from oracle import oracle as O
    if trie:
        o_s, o_p, o_t, o_n = O.beam_select_trie(
            si.row_offset_old, si.row_offset_new, si.score_old, si.logits, ti.sid,
            ti.trie.node_ptr, ti.trie.edge_tok, ti.trie.edge_child)
    else:
        o_s, o_p, o_t = O.beam_select(si.row_offset_old, si.row_offset_new, si.score_old,
                                      si.logits)
    g_s, g_p, g_t = (x.cpu().numpy() for x in (score_new, parent, token))
    same = (g_p == o_p) & (g_t == o_t)
    if trie:
        same &= node_new.cpu().numpy() == o_n
    err = float(np.abs(g_s[same].astype(np.float64) - o_s[same]).max()) if same.any() else None
    name = (I.TRIE_WORKLOADS if trie else I.SELECT_WORKLOADS)[cfg]["name"]
    return dict(si=si, name=name, nbytes=nbytes, launch_ms=launch_ms, trie=trie,
                n_sets=n_sets, R_new=R_new, rank_match=float(same.mean()), max_abs=err)


def select_entry(r) -> dict:
    gbs = r["nbytes"] / (r["launch_ms"] * 1e-3) / 1e9
    kern = "beam_select_trie" if r["trie"] else "beam_select"
    return {"workload": r["name"], "rows_in": int(r["si"].logits.shape[0]),
            "beams_kept": r["R_new"], "launch_us": r["launch_ms"] * 1e3,
            "value": r["R_new"] / (r["launch_ms"] * 1e-3), "unit": "beams-selected/s",
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS,
                         "traffic": recorded_traffic(r["name"], kern, SELECT_SOURCES),
                         "kernel": kern + " (select_rows + select_request)",
                         "algorithmic_bytes": r["nbytes"]},
            "input_copies_rotated": r["n_sets"],
            "spot_check": {"rank_match": r["rank_match"], "max_abs": r["max_abs"]}}


def step_entry(r) -> dict:
    gbs = r["nbytes"] / (r["launch_ms"] * 1e-3) / 1e9
    return {"workload": r["name"], "rows": r["st"].R_new, "launch_us": r["launch_ms"] * 1e3,
            "launch_us_reps": [round(x * 1e3, 3) for x in r["reps_ms"]],
            "value": r["st"].R_new / (r["launch_ms"] * 1e-3), "unit": "beam-rows/s",
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS,
                         "traffic": recorded_traffic(r["name"], "beam_step", STEP_SOURCES),
                         "kernel": "beam_step", "algorithmic_bytes": r["nbytes"]},
            "input_copies_rotated": r["n_sets"], "bit_exact": r["bit_exact"]}


def cpu_baseline(inp: I.Inputs, min_seconds: float = 10.0):
    """The fp64 oracle on the host cores: repeated passes over every row of
    the workload until about `min_seconds` of wall time have been spent."""
    from oracle import oracle as O
    n = O.default_threads()
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    rows = np.arange(inp.R)
    passes = 0
    t0 = time.perf_counter()
    while True:
        O.decode_attn_inputs(inp, rows=rows, n_threads=n)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": passes * inp.R / dt, "unit": "beam-rows/s", "cores": n, "kind": "oracle",
            "sample": f"fp64 oracle, {passes} passes over all {inp.R} rows x {inp.wl.Hq} heads "
                      f"of the same workload, {dt:.1f} s wall on {n} threads",
            "cpu_model": model, "host_cpus_visible": os.cpu_count(),
            "threads_note": "all CPUs of the process affinity, capped by OMP_NUM_THREADS "
                            "when set (the machine's allotment per GPU job)"}


def measured_peaks(reps: int = 5):
    """Sustained rates of this GPU from the probe kernels of libgr_peaks.so:
    bf16 MFMA TFLOP/s (independent 32x32x16 chains), streaming copy and read
    GB/s over 1 GiB buffers, and fp32 exp2 results per second.  Each figure
    is the best of `reps` timed launches (HIP events on the launch stream).
    They are reported beside the vendor peaks; the roofline fractions use
    the vendor peaks."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "shared_prefix_beam_amd", "libgr_peaks.so"))
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.gr_peak_mfma.argtypes = [P, I32, I32, P]
    lib.gr_peak_exp2.argtypes = [P, I32, I32, P]
    lib.gr_peak_copy.argtypes = [P, P, I64, I32, P]
    lib.gr_peak_read.argtypes = [P, I64, P, I32, P]
    for f in (lib.gr_peak_mfma, lib.gr_peak_exp2, lib.gr_peak_copy, lib.gr_peak_read):
        f.restype = ctypes.c_int
    stream = torch.cuda.current_stream()
    h = stream.cuda_stream
    grid = 2048                                    # 8 workgroups of 4 waves per compute unit
    out = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    n_bytes = 1 << 30
    src = torch.empty(n_bytes, dtype=torch.uint8, device="cuda").fill_(3)
    dst = torch.empty_like(src)

    def best_ms(call):
        call()
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            st = call()
            e1.record(stream)
            torch.cuda.synchronize()
            if st != 0:
                raise RuntimeError(f"probe launch failed ({st})")
            t = e0.elapsed_time(e1)
            best = t if best is None else min(best, t)
        return best

    iters_m, iters_e = 2000, 4000
    t_m = best_ms(lambda: lib.gr_peak_mfma(out.data_ptr(), grid, iters_m, h))
    t_e = best_ms(lambda: lib.gr_peak_exp2(out.data_ptr(), grid, iters_e, h))
    t_c = best_ms(lambda: lib.gr_peak_copy(src.data_ptr(), dst.data_ptr(), n_bytes // 16, grid, h))
    t_r = best_ms(lambda: lib.gr_peak_read(src.data_ptr(), n_bytes // 16, out.data_ptr(), grid, h))
    waves = grid * 4
    mfma_flops = waves * iters_m * 4 * 32768.0
    exps = grid * 256 * iters_e * 8.0
    res = {"bf16_mfma_TFLOPs": mfma_flops / (t_m * 1e-3) / 1e12,
           "hbm_copy_GBps": 2 * n_bytes / (t_c * 1e-3) / 1e9,
           "hbm_read_GBps": n_bytes / (t_r * 1e-3) / 1e9,
           "exp2_per_s": exps / (t_e * 1e-3),
           "note": "best of %d launches; vendor peaks (%.0f TFLOP/s bf16, %.0f GB/s HBM) "
                   "stay the roofline denominators" % (reps, PEAK_BF16_TFLOPS, PEAK_HBM_GBS)}
    del src, dst
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-baseline leg")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--only", choices=["primary", "secondary", "cfg1", "cfg2", "cfg3", "cfg4",
                                       "cfg5", "paged2", "paged4", "beam_step", "beam_step2",
                                       "select", "select2", "trie"],
                    help="time one workload only and print its launch time (profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run 10 device copies of 256 MiB (reference for HBM byte counters)")
    ap.add_argument("--peaks", action="store_true",
                    help="print only the measured sustained MFMA, HBM and exp2 rates")
    ap.add_argument("--write-profiles", metavar="DIR",
                    help="summarise rocprofv3 outputs under DIR into profiles/ (no GPU needed)")
    args = ap.parse_args()
    if args.write_profiles:
        write_profile_summaries(args.write_profiles)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path "
              "shards by request or KV head with no exchange, so run one process per GPU.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": 256 << 20, "launches": 10}), flush=True)
        return
    if args.peaks:
        print(json.dumps(measured_peaks()), flush=True)
        return
    if args.only in ("select", "select2", "trie"):
        r = (measure_select(TRIE_CFGS[0], args.steps, args.warmup, trie=True)
             if args.only == "trie" else
             measure_select(SELECT_CFGS[1 if args.only == "select2" else 0], args.steps,
                            args.warmup))
        print(json.dumps({"workload": r["name"], "launch_us": r["launch_ms"] * 1e3,
                          "rank_match": r["rank_match"]}), flush=True)
        return
    if args.only in ("beam_step", "beam_step2"):
        r = measure_step(STEP_CFGS[1 if args.only == "beam_step2" else 0], args.steps, args.warmup)
        print(json.dumps({"workload": r["name"], "launch_us": r["launch_ms"] * 1e3,
                          "bit_exact": r["bit_exact"]}), flush=True)
        return
    if args.only:
        paged = args.only.startswith("paged")
        cfg = {"primary": PRIMARY, "secondary": SECONDARY}.get(args.only)
        cfg = cfg if cfg is not None else int(args.only[5:] if paged else args.only[3:])
        r = measure(cfg, args.steps, args.warmup, page_size=PAGE_SIZE if paged else None, reps=1,
                    latency_calls=0, settle=lambda: measured_peaks(reps=2))
        print(json.dumps({"workload": r["inp"].wl.name, "launch_us": r["launch_ms"] * 1e3,
                          "ms_per_step": r["ms_per_step"]}), flush=True)
        return
    # the probe leg (about a second of GPU work) runs right before the
    # headline's warm-up: the timed steps then see a GPU whose clocks have
    # come up, not one that was idle during the host-side set-up
    peaks = {}
    prim = measure(PRIMARY, args.steps, args.warmup, settle=lambda: peaks.update(measured_peaks()))
    inp = prim["inp"]
    t_launch = prim["launch_ms"] * 1e-3
    achieved = prim["nbytes"] / t_launch / 1e9
    traffic = recorded_traffic(inp.wl.name)
    line = {
        "metric": METRIC,
        "value": inp.R / (prim["ms_per_step"] * 1e-3),
        "unit": "beam-rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": prim["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": inp.wl.name, "B": inp.B, "beams_per_request": int(inp.wl.W[0]),
                   "ctx_len": int(inp.ctx_len[0]), "beam_tokens": int(inp.beam_len[0]),
                   "Hq": inp.wl.Hq, "Hkv": inp.wl.Hkv, "D": inp.wl.D, "rows": inp.R,
                   "input_copies_rotated": prim["n_sets"]},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": kernel_of(prim["plan"]), "plan": prim["plan"],
                     "launch_us": prim["launch_ms"] * 1e3,
                     "launch_us_median": prim["launch_median_ms"] * 1e3,
                     "launch_us_min": prim["launch_min_ms"] * 1e3,
                     "algorithmic_bytes": prim["nbytes"]},
        "spot_check": {"max_abs": prim["spot_abs"], "lse_abs": prim["spot_lse"]},
    }
    sec = None
    if not args.no_secondary:
        sec = measure(SECONDARY, args.steps, args.warmup, settle=lambda: measured_peaks(reps=2))
        si = sec["inp"]
        tf = sec["flops"] / (sec["launch_ms"] * 1e-3) / 1e12
        line["secondary"] = {
            "workload": si.wl.name, "value": si.R / (sec["ms_per_step"] * 1e-3),
            "unit": "beam-rows/s", "ms_per_step": sec["ms_per_step"],
            "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS,
                         "traffic": recorded_traffic(si.wl.name),
                         "kernel": kernel_of(sec["plan"]), "plan": sec["plan"],
                         "launch_us": sec["launch_ms"] * 1e3,
                         "launch_us_median": sec["launch_median_ms"] * 1e3,
                         "launch_us_min": sec["launch_min_ms"] * 1e3,
                         "algorithmic_flops": sec["flops"],
                         "hbm_GBps": sec["nbytes"] / (sec["launch_ms"] * 1e-3) / 1e9},
            "spot_check": {"max_abs": sec["spot_abs"], "lse_abs": sec["spot_lse"]},
        }
    # every workload of the set, the two above included: rates at the median
    # of the repetitions, both roofline fractions, cold latency, spot check
    runs = {PRIMARY: prim}
    if sec is not None:
        runs[SECONDARY] = sec
    for c in sorted(I.WORKLOADS):
        if c not in runs:
            runs[c] = measure(c, args.steps, args.warmup)
    line["configs"] = [config_entry(c, runs[c]) for c in sorted(runs)]
    line["beam_step"] = [step_entry(measure_step(c, args.steps, args.warmup)) for c in STEP_CFGS]
    line["beam_select"] = [select_entry(measure_select(c, args.steps, args.warmup))
                           for c in SELECT_CFGS]
    line["beam_select_trie"] = [select_entry(measure_select(c, args.steps, args.warmup, trie=True))
                                for c in TRIE_CFGS]
    paged = []
    for cfg, dense in ((PRIMARY, prim), (SECONDARY, sec)):
        if dense is None:
            continue
        r = measure(cfg, args.steps, args.warmup, page_size=PAGE_SIZE)
        t = r["launch_ms"] * 1e-3
        paged.append({"workload": r["inp"].wl.name, "page_size": PAGE_SIZE,
                      "launch_us": r["launch_ms"] * 1e3,
                      "launch_us_median": r["launch_median_ms"] * 1e3,
                      "launch_us_min": r["launch_min_ms"] * 1e3,
                      "hbm_GBps": r["nbytes"] / t / 1e9, "TFLOPs": r["flops"] / t / 1e12,
                      "vs_dense_launch": dense["launch_ms"] / r["launch_ms"],
                      "vs_dense_launch_median": dense["launch_median_ms"] / r["launch_median_ms"],
                      "traffic": recorded_traffic(f"paged{PAGE_SIZE}_{r['inp'].wl.name}"),
                      "spot_check": {"max_abs": r["spot_abs"], "lse_abs": r["spot_lse"]}})
    line["paged"] = paged
    line["measured_peaks"] = peaks
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
