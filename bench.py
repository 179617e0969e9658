#!/usr/bin/env python3
"""Benchmark of the paged GQA attention hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic inputs:
slot mapping of the step's new tokens, then per layer the KV append and the
attention launches (prefill chunk and/or decode, with the split merge).
Inputs are resident in HBM before timing starts.

Default workload (c4): the Qwen3-8B-shaped decode step, 36 layers, batch 64
at context 4096 plus batch 13 at context 32768 (each with its own pools);
a step runs both batches.  Other configurations: --workload
c1|c2|c3|c4a|c4b|c5 (c5 cycles its six prefill-chunk offsets over steps).  Working sets under 1 GiB are rotated over
enough independent copies (>= 512 MiB in total) that the 256 MB Infinity
Cache cannot serve them.

Prints one JSON line (rank 0).  value = algorithmic HBM bytes of the step /
step time (GB/s); the roofline object reports the dominant kernel (the decode
attention call, measured with HIP events on the launch stream), the
cpu_baseline object the CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
GATE_CYCLES = 500_000          # GPU sleep queued before a timed launch (about 200 us)
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure
METRIC = "paged GQA decode: achieved HBM GB/s (% of peak) + decode tokens/s/GPU"


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="c4",
                   choices=["c1", "c2", "c3", "c4", "c4a", "c4b", "c5"])
    p.add_argument("--rotate-mib", type=int, default=512,
                   help="total bytes of rotated input copies for small working sets")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="CPU-oracle sample budget (0 disables the cpu_baseline leg)")
    p.add_argument("--no-events", action="store_true",
                   help="time steps only (no per-launch events), e.g. under a profiler")
    p.add_argument("--gate-cycles", type=int, default=GATE_CYCLES,
                   help="GPU sleep (cycles) queued before each launch timed by events in "
                        "graph mode")
    p.add_argument("--one-stream", action="store_true",
                   help="run everything on one stream: a step's parts one after the other, a "
                        "mixed step's decode after its chunk (default: each part of a step "
                        "on its own stream, and a mixed step's decode on a second stream, "
                        "concurrent with the chunk)")
    p.add_argument("--no-fuse", dest="fuse", action="store_false",
                   help="run each layer's append as its own call before the attention "
                        "(default: decode-only steps run pkv_attn_decode_append, or "
                        "pkv_attn_decode_append_int8 over int8 pages, and mixed steps "
                        "pkv_attn_prefill_decode_append, one call per layer)")
    p.add_argument("--no-mixed", dest="mixed", action="store_false",
                   help="run a mixed step's attention as pkv_attn_prefill_chunk + "
                        "pkv_attn_decode (default: one pkv_attn_prefill_decode call per "
                        "layer; int8 pages: pkv_attn_prefill_decode_int8)")
    p.add_argument("--kv", default="bf16", choices=["bf16", "int8"],
                   help="page format: bf16, or int8 codes with per-(slot, head) scales")
    p.add_argument("--kernels", action="store_true",
                   help="time the page-write kernels (append, int8 append, block copy, fused "
                        "norm+RoPE+append, slot mapping) by HIP-graph replay; one JSON line")
    p.add_argument("--eager", dest="graph", action="store_false",
                   help="launch every kernel from Python in the timed steps (default: capture "
                        "each distinct step in a HIP graph and time graph replays; per-kernel "
                        "times then come from graphs of one kernel's launches alone)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run plain 1 GiB device copies (counter calibration under rocprofv3)")
    p.add_argument("--write-trace-record", nargs=2, metavar=("KERNEL_TRACE_CSV", "LAUNCHES"),
                   help="CPU only: record the mean duration of the last LAUNCHES decode "
                        "dispatches (the launches the bench times one by one) from a "
                        "rocprofv3 --kernel-trace csv of this workload's bench command")
    p.add_argument("--write-traffic-record", nargs=4,
                   metavar=("COPY_FETCH_CSV", "COPY_WRITE_CSV", "FETCH_CSV", "WRITE_CSV"),
                   help="CPU only: build the decode traffic record from rocprofv3 --pmc "
                        "counter_collection.csv files (FETCH_SIZE / WRITE_SIZE of the copy "
                        "calibration and of this workload's run)")
    return p.parse_args()


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "decode_kernel_traffic.json")
TRACE_RECORD = os.path.join(ROOT, "profiles", "decode_kernel_trace.json")
DECODE_SOURCES = [os.path.join(ROOT, "paged_kv_gqa_pkv_amd", "csrc", f)
                  for f in ("decode_kernel.h", "decode.hip")]


def _decode_source_sha():
    """SHA-256 over the decode kernel's sources (its device code, then the
    launchers and planner)."""
    import hashlib
    h = hashlib.sha256()
    for path in DECODE_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(key):
    """HBM bytes per decode launch measured with rocprofv3 counters (FETCH_SIZE,
    WRITE_SIZE, scaled by the same counters on a plain copy) for this workload
    key ("c4", "c4-int8", ...), if the record was taken on the current decode
    kernel source; else None."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f).get("records", {}).get(key)
        sha = _decode_source_sha()
    except (OSError, ValueError):
        return None
    if not rec or rec.get("decode_source_sha256") != sha:
        return None
    return rec.get("traffic_bytes_per_launch")


def _record_key(args):
    return args.workload + ("" if args.kv == "bf16" else "-int8") + ("" if args.fuse else "-nofuse")


def measured_trace(args, bytes_per_launch):
    """The decode launches' mean duration in the committed rocprofv3 kernel
    trace of this workload's bench command (profiles/decode_kernel_trace.json),
    if it was taken on the current decode kernel source; else None."""
    try:
        with open(TRACE_RECORD) as f:
            rec = json.load(f).get("records", {}).get(_record_key(args))
        sha = _decode_source_sha()
    except (OSError, ValueError):
        return None
    if not rec or rec.get("decode_source_sha256") != sha:
        return None
    us = rec["avg_launch_us"]
    achieved = bytes_per_launch / (us * 1e-6) / 1e9
    return {"avg_launch_us": us, "achieved": round(achieved, 1),
            "frac": round(achieved / HBM_PEAK_GBS, 4), "launches": rec["launches"],
            "source": "rocprofv3 --kernel-trace, " + os.path.relpath(TRACE_RECORD, ROOT)}


def write_trace_record(args):
    """Mean duration of the last LAUNCHES decode dispatches of a rocprofv3
    kernel trace (csv) of the bench command: the gated eager pass that the
    bench's HIP events time launch by launch runs last."""
    import csv
    import statistics
    path, n = args.write_trace_record[0], int(args.write_trace_record[1])
    with open(path) as f:
        rows = [r for r in csv.DictReader(f) if "decode_kernel" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    last = rows[-n:]
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in last]
    per_grid = {}
    for r, d in zip(last, durs):
        per_grid.setdefault(r.get("Grid_Size", r.get("Grid_Size_X", "?")), []).append(d)
    rec = {"workload": _record_key(args), "decode_source_sha256": _decode_source_sha(),
           "launches": len(durs), "avg_launch_us": round(statistics.mean(durs), 2),
           "per_grid": {g: {"dispatches": len(v), "mean_us": round(statistics.mean(v), 2),
                            "median_us": round(statistics.median(v), 2)}
                        for g, v in sorted(per_grid.items())},
           "all_decode_dispatches": len(rows),
           "command": "rocprofv3 --kernel-trace --stats --output-format csv -- python3 bench.py "
                      f"--workload {args.workload} --kv {args.kv}" + ("" if args.fuse else " --no-fuse")}
    try:
        with open(TRACE_RECORD) as f:
            allrec = json.load(f)
    except (OSError, ValueError):
        allrec = {}
    allrec.setdefault("records", {})[rec["workload"]] = rec
    with open(TRACE_RECORD, "w") as f:
        json.dump(allrec, f, indent=1)
    print(json.dumps(rec), flush=True)


def write_traffic_record(args):
    """HBM bytes per decode launch from rocprofv3 counters (KiB per dispatch):
    each counter is scaled by true bytes / counted bytes of the plain 1 GiB
    copy, then the decode dispatches' mean FETCH and WRITE are summed."""
    import csv
    import hashlib
    import statistics

    def values(path, key):
        with open(path) as f:
            return [(r["Grid_Size"], float(r["Counter_Value"]))
                    for r in csv.DictReader(f) if key in r["Kernel_Name"]]

    copy_f, copy_w, dec_f, dec_w = args.write_traffic_record
    true_kib = (1 << 30) / 1024
    cf = [v for _, v in values(copy_f, "copyBuffer")]
    cw = [v for _, v in values(copy_w, "copyBuffer")]
    fetch_scale, write_scale = true_kib / statistics.mean(cf), true_kib / statistics.mean(cw)
    kname = "Int8Page" if args.kv == "int8" else "Bf16Page"
    df, dw = values(dec_f, kname), values(dec_w, kname)
    if not df or not dw:
        raise SystemExit(f"no {kname} decode dispatches in the counter files")
    per_grid = {}
    for grid in sorted({g for g, _ in df}):
        f = [v for g, v in df if g == grid]
        w = [v for g, v in dw if g == grid]
        per_grid[grid] = {"dispatches": len(f), "fetch_kib_mean": round(statistics.mean(f), 1),
                          "write_kib_mean": round(statistics.mean(w), 1),
                          "bytes": round(1024 * (statistics.mean(f) * fetch_scale +
                                                 statistics.mean(w) * write_scale))}
    traffic = round(1024 * (statistics.mean(v for _, v in df) * fetch_scale +
                            statistics.mean(v for _, v in dw) * write_scale))
    key = args.workload if args.kv == "bf16" else f"{args.workload}-int8"
    rec = {"kernel": f"decode_kernel<{kname}>", "workload": key,
           "decode_source_sha256": _decode_source_sha(), "traffic_bytes_per_launch": traffic,
           "fetch_scale": round(fetch_scale, 5), "write_scale": round(write_scale, 5),
           "copy_calibration": {"bytes_read": 1 << 30, "bytes_written": 1 << 30,
                                "fetch_kib_per_dispatch": cf, "write_kib_per_dispatch": cw},
           "per_grid": per_grid}
    try:
        with open(TRAFFIC_RECORD) as f:
            allrec = json.load(f)
    except (OSError, ValueError):
        allrec = {}
    allrec.setdefault("records", {})[key] = rec
    with open(TRAFFIC_RECORD, "w") as f:
        json.dump(allrec, f, indent=1)
    print(json.dumps(rec), flush=True)


def calibrate_copy():
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n,
                      "copies": 3}), flush=True)


# ---------------------------------------------------------------------------
# algorithmic work of a step (what the method must move / compute)
# ---------------------------------------------------------------------------

def decode_bytes(w, t, rows, kv="bf16"):
    """K/V of every token read once (pages shared by several tables counted
    once), q in and out, the table entries and lengths.  int8 pages: one byte
    per element plus a float32 K and V scale per (token, KV head)."""
    Hkv, D, Hq = w.Hkv, w.D, w.Hq
    per_token = 2 * Hkv * D * 2 if kv == "bf16" else 2 * Hkv * (D + 4)
    seen = {}
    table_bytes = 0
    for i in rows:
        n = int(t.context_lens[i])
        npg = (n + 15) // 16
        table_bytes += 4 * npg + 4
        for j in range(npg):
            page = int(t.block_tables[i, j])
            seen[page] = max(seen.get(page, 0), min(16, n - 16 * j))
    kv_tokens = sum(seen.values())
    return kv_tokens * per_token + len(rows) * 2 * Hq * D * 2 + table_bytes


def append_bytes(w, t, kv="bf16"):
    """Read the new bf16 K/V rows and the slot, write them into the pages (int8:
    the codes and a float32 scale per row)."""
    T = int(t.cu_new[-1])
    write = 2 * w.Hkv * w.D * 2 if kv == "bf16" else 2 * w.Hkv * (w.D + 4)
    return T * (2 * w.Hkv * w.D * 2 + write + 4)


def slot_bytes(w, t):
    T = int(t.cu_new[-1])
    return T * 12 + 4 * (len(w.seqs) * 2 + 1)


def prefill_work(w, t, kv="bf16"):
    """(bytes, causal FLOPs) of the prefill chunks: K/V of keys 0..o+T-1 once
    (int8 pages: codes and a float32 scale per key and KV head), q and out;
    FLOPs over visible (query, key) pairs only."""
    by, fl = 0, 0
    per_key = 2 * w.Hkv * (w.D * 2 if kv == "bf16" else w.D + 4)
    for i in w.prefill_seqs:
        s = w.seqs[i]
        o, T, n = s.pre_len, s.new_len, s.ctx
        by += n * per_key + 2 * T * w.Hq * w.D * 2 + 4 * ((n + 15) // 16)
        fl += 4 * w.D * w.Hq * (T * o + T * (T + 1) // 2)
    return by, fl


# ---------------------------------------------------------------------------

class Part:
    """One independent decode/mixed step shape with its own pools."""

    def __init__(self, w, t, plan, layers, bufs, copies, kv="bf16"):
        self.w, self.t, self.plan, self.layers, self.bufs, self.copies = w, t, plan, layers, bufs, copies
        self.kv = kv
        nd = len(w.decode_seqs)
        self.dec_bytes = decode_bytes(w, t, w.decode_seqs, kv) if nd else 0
        # the timed decode launch: a fused call also reads the step's new bf16
        # K/V rows in place of that position's pool rows, and writes those
        # rows into the pool (int8 pages: their codes and scales), which adds
        # the new rows' bf16 bytes in either format
        self.launch_bytes = self.dec_bytes + (nd * 2 * w.Hkv * w.D * 2 if plan.fused else 0)
        self.pre_bytes, self.pre_flops = prefill_work(w, t, kv)
        # the step's new K/V rows, as one fused mixed call writes them
        self.new_row_bytes = (int(t.cu_new[-1]) * 2 * w.Hkv * w.D * 2
                              if plan.fused and plan.mixed else 0)
        self.step_bytes = slot_bytes(w, t) + w.n_layers * (append_bytes(w, t, kv) +
                                                           self.dec_bytes + self.pre_bytes)


def _bufs(w, t, device):
    import torch
    from paged_kv_gqa_pkv_amd import synth as S
    npre = sum(w.seqs[i].new_len for i in w.prefill_seqs)
    qd = S.randn_bf16((len(w.decode_seqs), w.Hq, w.D), 77, device) if w.decode_seqs else None
    qp = S.randn_bf16((npre, w.Hq, w.D), 78, device) if npre else None
    T = int(t.cu_new[-1])
    return dict(qd=qd, qp=qp, kn=S.randn_bf16((T, w.Hkv, w.D), 79, device),
                vn=S.randn_bf16((T, w.Hkv, w.D), 80, device),
                od=torch.empty_like(qd) if qd is not None else None,
                op=torch.empty_like(qp) if qp is not None else None)


def _layers(w, t, rotate_mib, device, kv="bf16"):
    from paged_kv_gqa_pkv_amd import synth as S
    per_slot = 2 * w.Hkv * w.D * 2 if kv == "bf16" else 2 * w.Hkv * (w.D + 4)
    pool_bytes = w.num_blocks * 16 * per_slot
    copies = 1
    if w.n_layers * pool_bytes < (1 << 30):
        copies = max(1, -(-rotate_mib * (1 << 20) // (w.n_layers * pool_bytes)))
    fill = S.page_fill_counts(w, t)
    make = S.make_layer if kv == "bf16" else S.make_layer_int8
    layers = [make(w, t, l + 1000 * c, device=device, fill=fill)
              for c in range(copies) for l in range(w.n_layers)]
    return layers, copies


def build_parts(name, rotate_mib, device, kv="bf16", fuse=True, mixed=True):
    """Returns (parts, schedule): schedule(i) lists the parts step i runs."""
    import torch
    from paged_kv_gqa_pkv_amd import step as ST
    from paged_kv_gqa_pkv_amd import synth as S

    if name == "c4":
        parts = []
        for sub in ("c4a", "c4b"):
            w = S.workload(sub)
            t = S.make_tables(w)
            layers, copies = _layers(w, t, rotate_mib, device, kv)
            parts.append(Part(w, t, ST.plan_step(w, t, device=device, fused=fuse),
                              layers, _bufs(w, t, device), copies, kv))
        return parts, (lambda i: [0, 1])
    if name == "c5":
        base_w = S.workload("c5", 5)
        base_t = S.make_tables(base_w)
        layers, copies = _layers(base_w, base_t, rotate_mib, device, kv)
        parts = []
        for s in range(6):
            w = S.workload("c5", s)
            p = w.seqs[0]
            ctx = base_t.context_lens.clone(); ctx[0] = p.ctx
            new = torch.tensor([0, p.new_len] + [1] * len(w.decode_seqs), dtype=torch.int64)
            t = S.Tables(base_t.block_tables, ctx, torch.cumsum(new, 0).to(torch.int32),
                         torch.tensor([q.pre_len for q in w.seqs], dtype=torch.int32))
            # int8 pages: the append stays a launch of its own (no int8 form
            # of the one-launch append + attention)
            parts.append(Part(w, t, ST.plan_step(w, t, device=device,
                                                 fused=fuse and kv == "bf16", mixed=mixed),
                              layers, _bufs(w, t, device), copies, kv))
        return parts, (lambda i: [i % 6])
    w = S.workload(name)
    t = S.make_tables(w)
    layers, copies = _layers(w, t, rotate_mib, device, kv)
    return [Part(w, t, ST.plan_step(w, t, device=device, fused=fuse), layers,
                 _bufs(w, t, device), copies, kv)], (lambda i: [0])


WORKLOAD_TEXT = {
    "c4": "c4: Qwen3-8B-shaped decode step, 36 layers, Hq=32 Hkv=8 D=128, pages of 16: batch 64 "
          "at context 4096 (pool 16416 pages/layer) plus batch 13 at context 32768 (pool 26656 "
          "pages/layer, split-context path), one append per sequence per layer",
    "c5": "c5: mixed step, 512-query causal prefill chunk at offsets 0..2560 (cycled) of a "
          "3000-token prompt + 7 decode seqs ctx U[256,2048], 28 layers, Qwen3-0.6B attention",
}


def run(args):
    import torch
    from paged_kv_gqa_pkv_amd import binding as bd
    from paged_kv_gqa_pkv_amd import step as ST

    bd.load()
    device = "cuda"
    torch.cuda.set_device(0)
    parts, schedule = build_parts(args.workload, args.rotate_mib, device, args.kv, args.fuse,
                                  args.mixed)
    stream = torch.cuda.current_stream()
    # A mixed step's decode runs on a second stream, concurrent with the
    # chunk (both only read the pools after the append); default priority.
    dstream = torch.cuda.Stream()
    # The parts of a step (c4: the batch at context 4096 and the batch at
    # 32768, separate pools) are independent, so each runs on its own stream
    # (default priority); their workgroups then share the compute units
    # instead of each launch's last round running part-empty.
    pstreams = [torch.cuda.Stream() for _ in parts]
    use_events = not args.no_events
    dec_events, pre_events, mix_events = [], [], []

    def run_part(k, i, record, only=None, stream=None):
        pt = parts[k]
        plan, qb = pt.plan, pt.bufs
        c = i % pt.copies
        n_layers = pt.w.n_layers
        if only is None and plan.needs_slots:
            ST.slot_mapping(plan, stream=stream)
        for l in range(n_layers):
            d = pt.layers[c * n_layers + l]
            if plan.fused and not plan.mixed:
                # decode-only step: the layer's append and decode in one call
                if record:
                    if record == "gated":
                        torch.cuda._sleep(args.gate_cycles)
                    e0 = torch.cuda.Event(enable_timing=True); e0.record(stream)
                if pt.kv == "int8":
                    bd.pkv_attn_decode_append_int8(qb["od"], qb["qd"], qb["kn"], qb["vn"],
                                                   d.k_codes, d.v_codes, d.k_scales, d.v_scales,
                                                   plan.bt_decode, plan.ctx_decode,
                                                   plan.max_ctx_decode, plan.scale,
                                                   workspace=plan.workspace, stream=stream)
                else:
                    bd.pkv_attn_decode_append(qb["od"], qb["qd"], qb["kn"], qb["vn"], d.k_cache,
                                              d.v_cache, plan.bt_decode, plan.ctx_decode,
                                              plan.max_ctx_decode, plan.scale,
                                              workspace=plan.workspace, stream=stream)
                if record:
                    e1 = torch.cuda.Event(enable_timing=True); e1.record(stream)
                    dec_events.append((k, e0, e1, 1))
                continue
            if only is None and plan.fused:
                pass                  # the mixed call below appends the layer's rows itself
            elif only is None and pt.kv == "int8":
                bd.pkv_append_int8(qb["kn"], qb["vn"], plan.slot_mapping, d.k_codes, d.v_codes,
                                   d.k_scales, d.v_scales, stream=stream)
            elif only is None:
                bd.pkv_append(qb["kn"], qb["vn"], plan.slot_mapping, d.k_cache, d.v_cache,
                              stream=stream)
            if plan.mixed and only is None:
                # the chunk's and the decode's workgroups in one launch
                if record:
                    if record == "gated":
                        torch.cuda._sleep(args.gate_cycles)
                    e0 = torch.cuda.Event(enable_timing=True); e0.record(stream)
                if pt.kv == "int8":
                    bd.pkv_attn_prefill_decode_int8(
                        qb["op"], qb["qp"], plan.cu_q, plan.bt_prefill, plan.ctx_prefill,
                        plan.max_q_len, plan.max_ctx_prefill, qb["od"], qb["qd"],
                        plan.bt_decode, plan.ctx_decode, plan.max_ctx_decode, d.k_codes,
                        d.v_codes, d.k_scales, d.v_scales, plan.scale,
                        prefill_workspace=plan.prefill_workspace,
                        decode_workspace=plan.workspace, stream=stream)
                elif plan.fused:
                    bd.pkv_attn_prefill_decode_append(
                        qb["op"], qb["qp"], plan.cu_q, plan.bt_prefill, plan.ctx_prefill,
                        plan.max_q_len, plan.max_ctx_prefill, qb["od"], qb["qd"],
                        plan.bt_decode, plan.ctx_decode, plan.max_ctx_decode, qb["kn"],
                        qb["vn"], plan.slot_mapping, d.k_cache, d.v_cache, plan.scale,
                        prefill_workspace=plan.prefill_workspace,
                        decode_workspace=plan.workspace, stream=stream)
                else:
                    bd.pkv_attn_prefill_decode(qb["op"], qb["qp"], plan.cu_q, plan.bt_prefill,
                                               plan.ctx_prefill, plan.max_q_len,
                                               plan.max_ctx_prefill, qb["od"], qb["qd"],
                                               plan.bt_decode, plan.ctx_decode,
                                               plan.max_ctx_decode, d.k_cache, d.v_cache,
                                               plan.scale,
                                               prefill_workspace=plan.prefill_workspace,
                                               decode_workspace=plan.workspace, stream=stream)
                if record:
                    e1 = torch.cuda.Event(enable_timing=True); e1.record(stream)
                    mix_events.append((k, e0, e1, 1))
                continue
            if plan.n_prefill and only in (None, "prefill"):
                if record:
                    if record == "gated":
                        torch.cuda._sleep(args.gate_cycles)
                    e0 = torch.cuda.Event(enable_timing=True); e0.record(stream)
                if pt.kv == "int8":
                    bd.pkv_attn_prefill_chunk_int8(qb["op"], qb["qp"], plan.cu_q, d.k_codes,
                                                   d.v_codes, d.k_scales, d.v_scales,
                                                   plan.bt_prefill,
                                                   plan.ctx_prefill, plan.max_q_len,
                                                   plan.max_ctx_prefill, plan.scale,
                                                   workspace=plan.prefill_workspace,
                                                   stream=stream)
                else:
                    bd.pkv_attn_prefill_chunk(qb["op"], qb["qp"], plan.cu_q, d.k_cache,
                                              d.v_cache, plan.bt_prefill, plan.ctx_prefill,
                                              plan.max_q_len, plan.max_ctx_prefill, plan.scale,
                                              workspace=plan.prefill_workspace, stream=stream)
                if record:
                    e1 = torch.cuda.Event(enable_timing=True); e1.record(stream)
                    pre_events.append((k, e0, e1, 1))
            # the gated timing pass keeps one stream so that each kernel runs alone
            overlap = (bool(plan.n_prefill) and not args.one_stream and record != "gated"
                       and only is None)
            ds = dstream if overlap else stream
            if overlap:
                ev = torch.cuda.Event(); ev.record(stream); ds.wait_event(ev)
            if plan.n_decode and only in (None, "decode"):
                if record:
                    if record == "gated":
                        torch.cuda._sleep(args.gate_cycles)
                    e0 = torch.cuda.Event(enable_timing=True); e0.record(ds)
                if pt.kv == "int8":
                    bd.pkv_attn_decode_int8(qb["od"], qb["qd"], d.k_codes, d.v_codes,
                                            d.k_scales, d.v_scales, plan.bt_decode,
                                            plan.ctx_decode,
                                            plan.max_ctx_decode, plan.scale,
                                            workspace=plan.workspace, stream=ds)
                else:
                    bd.pkv_attn_decode(qb["od"], qb["qd"], d.k_cache, d.v_cache,
                                       plan.bt_decode, plan.ctx_decode, plan.max_ctx_decode,
                                       plan.scale, workspace=plan.workspace, stream=ds)
                if record:
                    e1 = torch.cuda.Event(enable_timing=True); e1.record(ds)
                    dec_events.append((k, e0, e1, 1))
            if overlap:
                ev = torch.cuda.Event(); ev.record(ds); stream.wait_event(ev)

    def one_step(i, record, only=None):
        ks = list(schedule(i))
        if len(ks) == 1 or args.one_stream or record == "gated" or only is not None:
            for k in ks:
                run_part(k, i, record, only, stream)
            return
        fork = torch.cuda.Event()
        fork.record(stream)
        for j, k in enumerate(ks):
            ps = stream if j == 0 else pstreams[j]
            if j:
                ps.wait_event(fork)
            run_part(k, i, record, only, ps)
        for j in range(1, len(ks)):
            join = torch.cuda.Event()
            join.record(pstreams[j])
            stream.wait_event(join)

    for i in range(args.warmup):
        one_step(i, False)
    torch.cuda.synchronize()
    if args.graph:
        # One graph per distinct step: the step pattern repeats with the
        # schedule's period times every part's number of rotated copies.
        period = 6 if args.workload == "c5" else 1
        for pt in parts:
            period = period * pt.copies // math.gcd(period, pt.copies)
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        graphs = []
        eager_stream = stream
        stream = cap
        with torch.cuda.stream(cap):
            for i in range(period):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    one_step(i, False)
                graphs.append(g)
        stream = eager_stream
        torch.cuda.synchronize()
        for g in graphs:          # one untimed replay each
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % period].replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        if use_events:
            # Per-launch durations: an eager pass after the timed replays, HIP
            # events around each launch on its stream, each (event, launch,
            # event) queued behind a GPU sleep so that the GPU never waits
            # for Python between them and the events bracket the kernel alone.
            for i in range(2 * period):
                one_step(i, "gated")
            torch.cuda.synchronize()
    else:
        t0 = time.perf_counter()
        for i in range(args.steps):
            one_step(i, use_events)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0

    total_bytes = sum(parts[k].step_bytes for i in range(args.steps) for k in schedule(i))
    dec_tokens = sum(len(parts[k].w.decode_seqs) for i in range(args.steps) for k in schedule(i))
    gbs = total_bytes / elapsed / 1e9
    roofline, extra = None, {}
    if dec_events:
        durs = [a.elapsed_time(b) * 1e-3 for (_, a, b, _) in dec_events]
        byts = [parts[k].launch_bytes * n for (k, _, _, n) in dec_events]
        n_launch = sum(n for (_, _, _, n) in dec_events)
        achieved = sum(byts) / sum(durs) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic(args.workload if args.kv == "bf16"
                                                else f"{args.workload}-int8"),
                    "kernel": (("decode_kernel<Int8Page, append> (pkv_attn_decode_append_int8)"
                                if parts[0].plan.fused else
                                "decode_kernel<Int8Page> (pkv_attn_decode_int8)")
                               if args.kv == "int8" else
                               "decode_kernel<Bf16Page, append> (pkv_attn_decode_append)"
                               if parts[0].plan.fused else "decode_kernel (pkv_attn_decode)"),
                    "avg_launch_us": round(sum(durs) / n_launch * 1e6, 2),
                    "bytes_per_launch": int(sum(byts) / n_launch),
                    "launches": n_launch,
                    "trace": measured_trace(args, sum(byts) / n_launch),
                    "timing": ("HIP events around each launch of an eager pass after the timed "
                               "graph replays, each launch queued behind a GPU sleep"
                               if args.graph else
                               "HIP events around each launch in the timed region")}
    if pre_events:
        durs = [a.elapsed_time(b) * 1e-3 for (_, a, b, _) in pre_events]
        fl = [parts[k].pre_flops * n for (k, _, _, n) in pre_events]
        n_launch = sum(n for (_, _, _, n) in pre_events)
        tflops = sum(fl) / sum(durs) / 1e12
        extra["prefill_mfma"] = {"bound": "mfma", "achieved": round(tflops, 2),
                                 "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                                 "avg_launch_us": round(sum(durs) / n_launch * 1e6, 2),
                                 "launches": n_launch,
                                 "kernel": ("prefill_kernel (pkv_attn_prefill_chunk)"
                                            if args.kv == "bf16" else
                                            "prefill_kernel<int8> (pkv_attn_prefill_chunk_int8)")}
    if mix_events:
        durs = [a.elapsed_time(b) * 1e-3 for (_, a, b, _) in mix_events]
        n_launch = sum(n for (_, _, _, n) in mix_events)
        # a fused call also writes the step's new rows (read from k_new in place
        # of the pool: the reads are counted above)
        byts = sum((parts[k].dec_bytes + parts[k].pre_bytes + parts[k].new_row_bytes) * n
                   for (k, _, _, n) in mix_events)
        fl = sum(parts[k].pre_flops * n for (k, _, _, n) in mix_events)
        achieved = byts / sum(durs) / 1e9
        mix_kernel = ("mixed_int8_kernel (pkv_attn_prefill_decode_int8)" if args.kv == "int8"
                      else "mixed_append_kernel (pkv_attn_prefill_decode_append)"
                      if parts[0].plan.fused else "mixed_kernel (pkv_attn_prefill_decode)")
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                    "kernel": mix_kernel,
                    "avg_launch_us": round(sum(durs) / n_launch * 1e6, 2),
                    "bytes_per_launch": int(byts / n_launch), "launches": n_launch,
                    "work": "the decode half's K/V, q/out and tables plus the chunk's keys "
                            "0..o+T-1, q and out, once each" + (
                                "; the step's new K/V rows written into their slots"
                                if parts[0].plan.fused else ""),
                    "trace": None,
                    "timing": ("HIP events around each launch of an eager pass after the timed "
                               "graph replays, each launch queued behind a GPU sleep"
                               if args.graph else
                               "HIP events around each launch in the timed region")}
        tflops = fl / sum(durs) / 1e12
        extra["prefill_mfma"] = {"bound": "mfma", "achieved": round(tflops, 2),
                                 "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                                 "avg_launch_us": round(sum(durs) / n_launch * 1e6, 2),
                                 "launches": n_launch,
                                 "kernel": mix_kernel +
                                           ": the chunk's causal FLOPs over the whole launch, "
                                           "decode included"}
    def pcts(events):
        # p10 / median / p90 of the timed launches, in us, per part of the step
        by = {}
        for (k, a, b, _) in events:
            by.setdefault(parts[k].w.name, []).append(a.elapsed_time(b) * 1e3)
        out = {}
        for name, d in by.items():
            d.sort()
            out[name] = [round(d[min(len(d) - 1, int(q * len(d)))], 2) for q in (0.1, 0.5, 0.9)]
        return out

    if roofline is not None and (dec_events or mix_events):
        roofline["launch_us_p10_p50_p90"] = pcts(dec_events or mix_events)
    if "prefill_mfma" in extra and (pre_events or mix_events):
        extra["prefill_mfma"]["launch_us_p10_p50_p90"] = pcts(pre_events or mix_events)
    w0 = parts[0].w
    cfg = {"workload": WORKLOAD_TEXT.get(args.workload, f"{args.workload}: {w0.description}"),
           "parts": [{"name": p.w.name, "layers": p.w.n_layers, "Hq": p.w.Hq, "Hkv": p.w.Hkv,
                      "head_dim": p.w.D, "decode_batch": len(p.w.decode_seqs),
                      "max_context": p.w.max_ctx, "pool_pages": p.w.num_blocks,
                      "rotated_copies": p.copies, "bytes_per_part_step": p.step_bytes,
                      "decode_splits": bd.pkv_decode_num_splits(
                          len(p.w.decode_seqs), p.w.Hq, p.w.Hkv, p.w.D,
                          p.plan.max_ctx_decode) if p.w.decode_seqs else 0}
                     for p in parts[:2]],
           "page_tokens": 16,
           "kv_pages": ("bf16" if args.kv == "bf16" else
                        "int8 codes + float32 (K, V) scale per slot and KV head"),
           "launch": (("HIP graph per step" if args.graph else "eager") + (
               ", each part on its own stream"
               if len(schedule(0)) > 1 and not args.one_stream
               else ", decode on a second stream concurrent with the chunk"
               if not args.one_stream and any(p.plan.n_prefill and p.plan.n_decode and
                                              not p.plan.mixed for p in parts)
               else ", one stream") + (
               "; decode-only layers: one fused append + decode call"
               if any(p.plan.fused and not p.plan.mixed for p in parts) else "") + (
               "; mixed layers: one launch for the append, the chunk and the decode"
               if any(p.plan.mixed and p.plan.fused for p in parts) else
               "; mixed layers: append, then one launch for the chunk and the decode"
               if any(p.plan.mixed for p in parts) else ""))}
    out = {"metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(1e3 * elapsed / args.steps, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if args.kv == "bf16" else "int8 pages, bf16 q/out",
           "data": "synthetic (seeded N(0,1) bf16, random page placement)",
           "config": cfg, "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
           "decode_tokens_per_s": round(dec_tokens / elapsed, 1), "roofline": roofline}
    out.update(extra)
    return out, parts


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _host_threads():
    """The host cores this process may use: its affinity set, capped by the
    thread count the environment grants (OMP_NUM_THREADS, when set)."""
    n = len(os.sched_getaffinity(0))
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        cap = 0
    return min(n, cap) if cap > 0 else n


def _oracle_sample(parts, budget, threads):
    """Seconds per full step of the oracle (as it stands) with BLAS limited to
    `threads`: one layer of each part of the step (slot mapping, append,
    attention), repeated until the part's share of the budget is spent, scaled
    to all layers.  Returns (seconds per step, description)."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from oracle import pkv_int8_oracle as Q
    from oracle import pkv_oracle as O
    from paged_kv_gqa_pkv_amd import synth as S

    def u16(x):
        return x.cpu().view(torch.int16).numpy().view(np.uint16)

    per_step, desc = 0.0, []
    share = budget / len(parts[:2])
    for pt in parts[:2]:
        w, t = pt.w, pt.t
        if pt.kv == "int8":
            d = S.make_layer_int8(w, t, 0)
            kc0, vc0 = d.k_codes.numpy(), d.v_codes.numpy()
            ks0, vs0 = d.k_scales.numpy(), d.v_scales.numpy()
        else:
            d = S.make_layer(w, t, 0)
            kc0, vc0 = u16(d.k_cache), u16(d.v_cache)
        kn, vn = u16(d.k_new), u16(d.v_new)
        qd = u16(d.q_decode) if d.q_decode is not None else None
        qp = u16(d.q_prefill) if d.q_prefill is not None else None
        bt, ctx = t.block_tables.numpy().tolist(), t.context_lens.numpy().tolist()
        cu = t.cu_new.numpy().tolist()
        npre = len(w.prefill_seqs)
        scale = O.default_scale(w.D)
        reps = 0
        with threadpool_limits(limits=threads):
            t0 = time.perf_counter()
            while True:
                slots = O.slot_ref(bt, cu, ctx)
                if pt.kv == "int8":
                    kc, vc, ks, vs = Q.append_int8_ref(kc0, vc0, ks0, vs0, kn, vn, slots)
                    if npre:
                        Q.prefill_int8_ref(qp, S.prefill_cu(w).numpy().tolist(), kc, ks, vc, vs,
                                           bt[:npre], ctx[:npre], scale)
                    if w.decode_seqs:
                        Q.decode_int8_ref(qd, kc, ks, vc, vs, bt[npre:], ctx[npre:], scale)
                else:
                    kc, vc = O.append_ref(kc0, vc0, kn, vn, slots)
                    if npre:
                        O.prefill_ref(qp, S.prefill_cu(w).numpy().tolist(), kc, vc, bt[:npre],
                                      ctx[:npre], scale)
                    if w.decode_seqs:
                        O.decode_ref(qd, kc, vc, bt[npre:], ctx[npre:], scale)
                reps += 1
                used = time.perf_counter() - t0
                if used >= share:
                    break
        per_step += used / reps * w.n_layers
        desc.append(f"{w.name}: {reps} x 1 of {w.n_layers} layers in {used:.1f} s")
    return per_step, "; ".join(desc)


def cpu_baseline(args, parts):
    """The CPU oracle (fp64 numpy, as it stands) on a bounded sample of the
    same workload, scaled to the whole step: on the host cores this process
    may use (BLAS threads = that count), and on one thread for reference."""
    step_b = sum(pt.step_bytes for pt in parts[:2])
    threads = _host_threads()
    per_step, desc = _oracle_sample(parts, args.cpu_seconds, threads)
    per_step1, desc1 = _oracle_sample(parts, args.cpu_seconds / 2, 1)
    return {"value": round(step_b / per_step / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "cpu": _cpu_model(),
            "sample": f"{desc} on {threads} host threads (fp64 numpy, BLAS threads {threads}), "
                      f"scaled to {per_step:.1f} s per full step",
            "value_1_thread": round(step_b / per_step1 / 1e9, 4),
            "sample_1_thread": f"{desc1} on 1 thread, scaled to {per_step1:.1f} s per full step"}


def _graph_time(fn, n_variants, reps=40):
    """GPU time per call: capture calls fn(0..k-1) (k >= 8, cycling over the
    rotated inputs) in one HIP graph, replay it, HIP events around the replays."""
    import torch
    k = max(8, n_variants)
    for i in range(k):
        fn(i)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for i in range(k):
                fn(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    r = max(2, reps // k)
    e0.record()
    for _ in range(r):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / (r * k)


def kernel_bench():
    """Per-kernel GPU time of the page-write kernels on synthetic inputs of the
    pages' shapes (Qwen3-8B-shaped heads: Hq 32, Hkv 8, D 128), each call on a
    different copy of its inputs so the 256 MB MALL cannot serve them.
    Algorithmic bytes: what the method must read and write once."""
    import torch
    from paged_kv_gqa_pkv_amd import binding as bd
    from paged_kv_gqa_pkv_amd import synth as S

    bd.load()
    torch.cuda.set_device(0)
    dev = "cuda"
    Hq, Hkv, D = 32, 8, 128
    out = {}

    def line(name, sec, nbytes, note):
        out[name] = {"us": round(sec * 1e6, 2), "bytes": int(nbytes),
                     "GBs": round(nbytes / sec / 1e9, 1),
                     "frac_of_8TBs": round(nbytes / sec / 1e9 / HBM_PEAK_GBS, 4), "work": note}

    # bf16 and int8 append: 65536 tokens into distinct slots of a 4096-page pool
    n_tok, nb, copies = 65536, 4096, 4
    sets = [S.bulk_append_inputs(n_tok, nb, Hkv, D, seed=300 + c, device=dev) for c in range(copies)]
    sets = [(sl.to(dev), kn, vn, pk, pv) for sl, kn, vn, pk, pv in sets]
    sec = _graph_time(lambda i: bd.pkv_append(sets[i % copies][1], sets[i % copies][2],
                                               sets[i % copies][0], sets[i % copies][3],
                                               sets[i % copies][4]), copies)
    line("append_bf16", sec, n_tok * (2 * 2 * Hkv * D * 2 + 4),
         f"{n_tok} tokens: read K/V rows and slot, write K/V rows")
    i8 = [(torch.zeros((nb, 16, Hkv, D), dtype=torch.int8, device=dev),
           torch.zeros((nb, 16, Hkv, D), dtype=torch.int8, device=dev),
           torch.zeros((nb, Hkv, 16), dtype=torch.float32, device=dev),
           torch.zeros((nb, Hkv, 16), dtype=torch.float32, device=dev)) for _ in range(copies)]
    sec = _graph_time(lambda i: bd.pkv_append_int8(sets[i % copies][1], sets[i % copies][2],
                                                    sets[i % copies][0], *i8[i % copies]), copies)
    line("append_int8", sec, n_tok * (2 * Hkv * D * 2 + 2 * Hkv * (D + 4) + 4),
         f"{n_tok} tokens: read bf16 K/V rows and slot, write codes and scales")
    del sets, i8
    # block copy: 1024 (src, dst) pairs in all 36 layers of a layered K and V pool
    L, nbc, pairs = 36, 4096, 1024
    kp = torch.empty((L, nbc, 16, Hkv, D), dtype=torch.bfloat16, device=dev)
    vp = torch.empty_like(kp)
    perm = torch.randperm(nbc, generator=torch.Generator().manual_seed(5))
    srcs = [perm[:pairs].to(torch.int32).to(dev), perm[pairs:2 * pairs].to(torch.int32).to(dev)]
    dsts = [perm[2 * pairs:3 * pairs].to(torch.int32).to(dev),
            perm[3 * pairs:4 * pairs].to(torch.int32).to(dev)]
    sec = _graph_time(lambda i: bd.pkv_copy_blocks(srcs[i % 2], dsts[i % 2], kp, vp,
                                                   layered=True), 2)
    line("copy_blocks", sec, pairs * L * 2 * Hkv * 16 * D * 2 * 2,
         f"{pairs} block pairs x {L} layers, K and V: read and write each block")
    del kp, vp
    # fused q/k RMSNorm + RoPE + append: 8192 decode tokens (one per sequence)
    B = 8192
    cos = (torch.rand((32768, D), device=dev) * 2 - 1).to(torch.bfloat16)
    sin = (torch.rand((32768, D), device=dev) * 2 - 1).to(torch.bfloat16)
    nbf = B * 4 + 16
    ctx = torch.randint(1, 4 * 16, (B,), generator=torch.Generator().manual_seed(6)).to(torch.int32)
    bt = torch.randperm(nbf, generator=torch.Generator().manual_seed(7))[:B * 4].view(B, 4)
    bt, ctx = bt.to(torch.int32).to(dev), ctx.to(dev)
    cu = torch.arange(B + 1, dtype=torch.int32, device=dev)
    fz = []
    for c in range(2):
        fz.append(dict(q=S.randn_bf16((B, Hq, D), 400 + c, dev), k=S.randn_bf16((B, Hkv, D), 410 + c, dev),
                       v=S.randn_bf16((B, Hkv, D), 420 + c, dev),
                       qo=torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev),
                       kc=torch.empty((nbf, 16, Hkv, D), dtype=torch.bfloat16, device=dev),
                       vc=torch.empty((nbf, 16, Hkv, D), dtype=torch.bfloat16, device=dev)))
    w = torch.ones(D, dtype=torch.bfloat16, device=dev)
    sm = torch.empty(B, dtype=torch.int32, device=dev)
    sec = _graph_time(lambda i: bd.pkv_qk_norm_rope_append(
        fz[i % 2]["qo"], fz[i % 2]["q"], fz[i % 2]["k"], fz[i % 2]["v"], w, w, cos, sin, bt, cu, ctx,
        fz[i % 2]["kc"], fz[i % 2]["vc"], 1e-6, slot_mapping=sm), 2)
    per_tok = 2 * Hq * D * 2 + 2 * Hkv * D * 2 * 2 + 2 * D * 2 + 4 * 3
    line("qk_norm_rope_append", sec, B * per_tok,
         f"{B} tokens: read q, k, v rows and the cos/sin rows of their positions, "
         "write rotated q and the K/V rows, slot and table entries")
    sec = _graph_time(lambda i: bd.pkv_slot_mapping(sm, bt, cu, ctx), 1)
    line("slot_mapping", sec, B * 12, f"{B} tokens: read table entry and lengths, write slot")
    del fz
    # what a plain read+write stream reaches on this part: the ceiling for the
    # append and copy kernels, which read and write every byte once
    src = torch.ones(1 << 29, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    sec = _graph_time(lambda i: dst.copy_(src), 1)
    line("device_copy", sec, 2 << 29, "torch copy of 512 MiB: read and write each byte once")
    del src, dst
    # what a tuned library GEMM reaches on this part in bf16 (hipBLASLt
    # through torch.mm, timed eagerly with events): the box's practical
    # matrix-core ceiling, beside the 2.5 PFLOP/s figure
    ga = S.randn_bf16((8192, 8192), 11, dev)
    gb = S.randn_bf16((8192, 8192), 12, dev)
    gc = torch.empty((8192, 8192), dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        torch.mm(ga, gb, out=gc)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(20):
        torch.mm(ga, gb, out=gc)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / 20
    gemm_tflops = 2 * 8192 ** 3 / sec / 1e12
    out["bf16_gemm_8192"] = {"us": round(sec * 1e6, 2), "TFLOPs": round(gemm_tflops, 1),
                             "frac_of_bf16_peak": round(gemm_tflops / BF16_PEAK_TFLOPS, 4),
                             "work": "torch.mm of two 8192 x 8192 bf16 matrices, "
                                     "1099.5 GFLOP: the box's library GEMM ceiling"}
    del ga, gb, gc
    # chunked prefill on a large chunk: 2048 queries at positions 6144..8191
    # (Qwen3-8B heads: 64 row tiles of 128 rows per KV head, 512 in all, which
    # the planner cuts into 2 key splits), bf16 and int8 pages; reported
    # against the bf16 MFMA peak
    c = S.large_chunk_inputs(dev)
    T, o, n = c["T"], c["offset"], c["n"]
    btp, ctxp, cuq, qp = c["block_tables"], c["context_lens"], c["cu_q"], c["q"]
    op = torch.empty_like(qp)
    nws = bd.pkv_prefill_workspace_bytes(1, T, Hq, Hkv, D, n)
    ws = torch.zeros(max(nws, 1), dtype=torch.uint8, device=dev)
    flops = 4 * D * Hq * (T * o + T * (T + 1) // 2)
    sec = _graph_time(lambda i: bd.pkv_attn_prefill_chunk(op, qp, cuq, c["k_cache"], c["v_cache"],
                                                          btp, ctxp, T, n, D ** -0.5,
                                                          workspace=ws), 1)
    out["prefill_2048x8192"] = {"us": round(sec * 1e6, 2), "TFLOPs": round(flops / sec / 1e12, 1),
                                "frac_of_bf16_peak": round(flops / sec / 1e12 / BF16_PEAK_TFLOPS, 4),
                                "frac_of_gemm": round(flops / sec / 1e12 / gemm_tflops, 4),
                                "work": f"one {T}-query causal chunk at positions {o}..{n - 1}, "
                                        f"Hq {Hq} Hkv {Hkv}, {flops / 1e9:.1f} GFLOP"}
    sec = _graph_time(lambda i: bd.pkv_attn_prefill_chunk_int8(
        op, qp, cuq, c["k_codes"], c["v_codes"], c["k_scales"], c["v_scales"], btp, ctxp, T, n,
        D ** -0.5, workspace=ws), 1)
    out["prefill_int8_2048x8192"] = {"us": round(sec * 1e6, 2),
                                     "TFLOPs": round(flops / sec / 1e12, 1),
                                     "frac_of_bf16_peak": round(flops / sec / 1e12 / BF16_PEAK_TFLOPS, 4),
                                     "frac_of_gemm": round(flops / sec / 1e12 / gemm_tflops, 4),
                                     "work": "the same chunk over int8 pages"}
    del c
    # sliding-window ring paging, a window of 4096 tokens (Module 04 page,
    # section 4): the batch-64 decode of Qwen3-8B heads at position 32768,
    # each sequence reading its last 4096 tokens through a 256-page ring
    # (two pool copies, alternated), and one 512-query chunk at positions
    # 32768..33279 through the first sequence's ring
    W, n_r, Br = 4096, 32768, 64
    rpages = W // 16
    npool = Br * rpages + 16
    pools = [(S.randn_bf16((npool, 16, Hkv, D), 440 + c, dev),
              S.randn_bf16((npool, 16, Hkv, D), 450 + c, dev)) for c in range(2)]
    btr = (torch.randperm(npool, generator=torch.Generator().manual_seed(9))[:Br * rpages]
           .view(Br, rpages).to(torch.int32).to(dev))
    ctxr = torch.full((Br,), n_r, dtype=torch.int32, device=dev)
    qd = S.randn_bf16((Br, Hq, D), 460, dev)
    od = torch.empty_like(qd)
    nwd = bd.pkv_decode_workspace_bytes(Br, Hq, Hkv, D, min(n_r, W))
    wsd = torch.zeros(max(nwd, 1), dtype=torch.uint8, device=dev) if nwd else None
    sec = _graph_time(lambda i: bd.pkv_attn_decode_ring(od, qd, pools[i % 2][0], pools[i % 2][1],
                                                        btr, ctxr, n_r, W, D ** -0.5,
                                                        workspace=wsd), 2)
    line("decode_ring_w4096", sec, Br * (W * 2 * Hkv * D * 2 + 2 * Hq * D * 2 + 4 * rpages + 4),
         f"{Br} sequences at position {n_r}, window {W}: read the window's K/V once, q, "
         "the ring table and length, write out")
    T, n_p = 512, n_r + 512
    qr = S.randn_bf16((T, Hq, D), 470, dev)
    orr = torch.empty_like(qr)
    cur = torch.tensor([0, T], dtype=torch.int32, device=dev)
    ctxp1 = torch.tensor([n_p], dtype=torch.int32, device=dev)
    nwp = bd.pkv_prefill_workspace_bytes(1, T, Hq, Hkv, D, min(n_p, W + 64))
    wsp = torch.zeros(max(nwp, 1), dtype=torch.uint8, device=dev) if nwp else None
    flops = 4 * D * Hq * (T * (W - T) + T * (T + 1) // 2)
    sec = _graph_time(lambda i: bd.pkv_attn_prefill_chunk_ring(
        orr, qr, cur, pools[i % 2][0], pools[i % 2][1], btr[:1], ctxp1, T, n_p, W, D ** -0.5,
        workspace=wsp), 2)
    out["prefill_ring_w4096"] = {"us": round(sec * 1e6, 2), "TFLOPs": round(flops / sec / 1e12, 1),
                                 "frac_of_bf16_peak": round(flops / sec / 1e12 / BF16_PEAK_TFLOPS, 4),
                                 "frac_of_gemm": round(flops / sec / 1e12 / gemm_tflops, 4),
                                 "work": f"one {T}-query chunk at positions {n_r}..{n_p - 1} over a "
                                         f"ring of {W} tokens, Hq {Hq} Hkv {Hkv}, "
                                         f"{flops / 1e9:.1f} GFLOP"}
    del pools
    # decode at group sizes 2, 4 and 8 (Hkv 8, Hq 8 G; Qwen3-0.6B-, Qwen3-8B-
    # and 70B-class head ratios): a batch of 64 at context 4096, pages placed
    # at random, two pool copies alternated; bf16 pages run the v_dot2 policy
    # below G = 8 and the matrix-core one at G = 8, int8 pages the
    # matrix-core one throughout
    Bg, ng = 64, 4096
    gpages = ng // 16
    npg = Bg * gpages + 16
    btg = (torch.randperm(npg, generator=torch.Generator().manual_seed(19))[:Bg * gpages]
           .view(Bg, gpages).to(torch.int32).to(dev))
    ctxg = torch.full((Bg,), ng, dtype=torch.int32, device=dev)
    for kv in ("bf16", "int8"):
        if kv == "bf16":
            gp = [(S.randn_bf16((npg, 16, Hkv, D), 480 + 2 * c, dev),
                   S.randn_bf16((npg, 16, Hkv, D), 481 + 2 * c, dev)) for c in range(2)]
            per_tok = 2 * Hkv * D * 2
        else:
            gp = [S.int8_pools(npg, Hkv, D, 484 + 3 * c, dev) for c in range(2)]
            per_tok = 2 * Hkv * (D + 4)
        for G in (2, 4, 8):
            Hqg = Hkv * G
            qg = S.randn_bf16((Bg, Hqg, D), 490 + G, dev)
            og = torch.empty_like(qg)
            nw = bd.pkv_decode_workspace_bytes(Bg, Hqg, Hkv, D, ng)
            wsg = torch.zeros(max(nw, 1), dtype=torch.uint8, device=dev) if nw else None
            if kv == "bf16":
                fn = lambda i: bd.pkv_attn_decode(og, qg, gp[i % 2][0], gp[i % 2][1], btg, ctxg,
                                                  ng, D ** -0.5, workspace=wsg)
            else:
                fn = lambda i: bd.pkv_attn_decode_int8(og, qg, *gp[i % 2], btg, ctxg, ng,
                                                       D ** -0.5, workspace=wsg)
            sec = _graph_time(fn, 2)
            line(f"decode_{kv}_g{G}", sec,
                 Bg * (ng * per_tok + 2 * Hqg * D * 2 + 4 * gpages + 4),
                 f"batch {Bg} at context {ng}, Hq {Hqg} Hkv {Hkv}, {kv} pages: read the K/V "
                 "once, q, the table and length, write out")
        del gp
    return {"kernels": out, "note": "GPU time per call from HIP-graph replay of >= 8 calls "
                                   "(the library GEMM: 20 eager calls between HIP events)"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if args.write_traffic_record:
        write_traffic_record(args)
        return
    if args.write_trace_record:
        write_trace_record(args)
        return
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.kernels:
        print(json.dumps(kernel_bench()), flush=True)
        return
    out, parts = run(args)
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(args, parts)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
