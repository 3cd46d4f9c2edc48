#!/usr/bin/env python3
"""Benchmark: the bit-exact delta refit hot path on one MI355X.

Headline workload, the largest configuration that runs both encode and apply
on one GPU: a Qwen3-30B-A3B-shaped MoE checkpoint (hidden 2048, 48 layers,
128 experts of FFN 768, 32 q / 4 kv heads x 128, vocab 151936; 30.5 B BF16
parameters and 0.9 GB of fp32 block scales, 62.0 GB canonical) trained with
expert parallelism 8.  5 % of the stored values change: 1 % of the rows of
every 2-D tensor change at 100 % (hot rows), the expert tensors are
block-scaled (one fp32 scale per 128 elements, and a changed scale changes
its whole block, which goes out as overwrite records), the rest is uniform
(+-1 BF16 ulp).  Inputs are synthetic and seeded, generated on the GPU;
nothing is read from disk.

One step = one pass of the whole hot path:
  encode (DELTA)   bit-diff + projection + routing + compaction + records
                   (staged), then the fix-up pass (offsets, records moved
                   into place)
  apply            the DELTA stream in place on the receiver's canonical tensors
  encode (RETRY)   the whole change set as overwrites
  retry            the RETRY stream re-applied as overwrites
value = canonical bytes scanned per step / step time (GB/s).

The same JSON line carries every other configuration under "configs" (one
4096x4096 tensor; Llama-8B TP=4; Qwen3-30B EP=8 at Beta(2,60) rates with a
3 % mean; the 240 GB receiver share, apply and retry only), each op with its
main kernel's roofline, and the CPU baseline: the oracle on one thread over a
bounded sample of the headline workload, and the oracle over the whole
headline workload on the host cores this process may use, which also
compares every record of both streams with the GPU's.

Prints one JSON line.  --gpus above 1 is refused: the path runs on one GPU.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
TARGET_FRAC = 0.70
LINE = 128   # bytes an apply reads per touched line (L2 line fill)
SECTOR = 32  # bytes an apply writes back per dirty sector (the L2 writes dirty 32-byte sectors)
HEADLINE = "qwen3_30b_hot_block_scaled"


def workloads():
    """(key, layout constructor or None, description) in the order they run."""
    from bit_exact_xor_amd import synth
    return [
        (HEADLINE, synth.config4_layout,
         "Qwen3-30B-A3B-shaped MoE checkpoint (30.5 B BF16 + 0.9 GB fp32 block scales, 62.0 GB), EP=8 trainer "
         "shards, 5% of stored values changed: hot rows (1% of the rows of every 2-D tensor at 100%), expert "
         "tensors block-scaled (one fp32 scale per 128 elements; changed scales send their blocks as "
         "overwrite records), the rest uniform +-1 ulp"),
        ("llama8b_tp4", synth.llama_layout,
         "Llama-8B-shaped BF16 checkpoint (16.1 GB), TP=4 trainer shards, fused QKV -> overwrite, 1% uniform "
         "+-1 ulp changes"),
        ("tensor_4096x4096", synth.config1_layout,
         "one 4096x4096 BF16 tensor (33.5 MB), identity projection, 1.00% of values changed by "
         "BF16(fp32(old) + lr * noise) plus 64 forced +0 <-> -0 flips, all XOR"),
        ("qwen3_30b_ep8_beta", synth.config3_layout,
         "Qwen3-30B-A3B-shaped MoE checkpoint (61.1 GB), EP=8 trainer shards, per-tensor change rates "
         "Beta(2,60) rescaled to a 3% mean, +-1 ulp"),
        ("receiver_share_240GB", synth.config5_layout,
         "one GPU's receiver share of a 1T model: 6812 x [7168,2048] BF16 (200 GB) at 3% + 5450 x [7168,1024] "
         "uint8 NVFP4-packed (40 GB) at 0.085% of bytes; apply and overwrite retry only"),
    ]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle legs (the one-thread sample and the whole-workload pass)")
    ap.add_argument("--cpu-reps", type=int, default=3, help="oracle steps timed on the one-thread sample")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the measurements outside the step (partial retry, RETRY from DELTA, index "
                         "lists, receiver layout, pipelined transfer, staging sizes, graph replay); for "
                         "profiler runs")
    ap.add_argument("--only", default=None, metavar="KEYS",
                    help="comma-separated workload keys to run (the first one run is the line's headline); "
                         "for profiler runs")
    ap.add_argument("--copy-probe", type=float, default=0.0, metavar="GIB",
                    help="only run a plain device copy of this many GiB, 3 times (counter calibration)")
    ap.add_argument("--pmc-report", metavar="DIR",
                    help="summarise rocprofv3 FETCH_SIZE / WRITE_SIZE runs found under DIR (of the workload "
                         "named by --only, default the headline) and exit")
    ap.add_argument("--pmc-dump", metavar="DIR",
                    help="per-kernel averages of every counter in the rocprofv3 runs under DIR/pmc_*; exit")
    ap.add_argument("--lists-cfg5", action="store_true",
                    help="only compare the bitmap and index-list streams on the receiver share's NVFP4 region "
                         "(40 GB at 0.085 %% bytes) and a 29 GB slice of its BF16 region (3 %%); one JSON line")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.pmc_report:
        print(pmc_report(args.pmc_report, (args.only or HEADLINE).split(",")[0]))
        return
    if args.pmc_dump:
        print(pmc_dump(args.pmc_dump))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py: --gpus {args.gpus}: the library runs the hot path on one GPU only "
              "(no cross-GPU sharding or collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_exact_xor_amd import dcr

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dcr.load_library()
    dev = "cuda"
    torch.cuda.set_device(0)
    if args.copy_probe:
        n = int(args.copy_probe * (1 << 30)) // 4
        src = torch.ones(n, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": 4 * n, "reps": 3}), flush=True)
        return
    if args.lists_cfg5:
        print(json.dumps(lists_cfg5(dev)), flush=True)
        return

    only = args.only.split(",") if args.only else None
    t_all = time.time()
    results = {}
    head_key = None
    for key, make, desc in workloads():
        if only and key not in only:
            continue
        head = head_key is None
        if head:
            head_key = key
        log(f"workload {key} ({'headline' if head else 'configs'})")
        if key == "receiver_share_240GB":
            results[key] = run_receiver_share(desc, dev, args)
        else:
            results[key] = run_workload(key, make, desc, dev, args, headline=head)
        gc.collect()
        torch.cuda.empty_cache()
        log(f"workload {key} done ({time.time() - t_all:.0f}s)")
    if head_key is None:
        raise SystemExit("no workload selected")
    h = results[head_key]
    out = {
        "metric": "encode & apply GB/s of BF16 weights scanned; % of MI355X HBM peak",
        "value": h["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u16",
        "data": "synthetic, seeded (GPU-generated shards)",
        "config": {"workload": h["workload"], **h["config"]},
        "ops": h["ops"],
        "roofline": h["roofline"],
        "target": {"hbm_frac": TARGET_FRAC, **h["target"]},
        "streams": h["streams"],
        "checks": h["checks"],
        "cpu_baseline": h.get("cpu_baseline"),
        "ceiling": h.get("ceiling"),
        "configs": {k: v for k, v in results.items() if k != head_key},
        "wall_s": round(time.time() - t_all, 1),
    }
    for k in ("staging", "hot_rows", "extras"):
        if k in h:
            out[k] = h[k]
    print(json.dumps(out), flush=True)


# ----------------------------------------------------------------- helpers

def _contiguous(lay):
    """Whether every canonical tensor is one contiguous run of one shard."""
    for g in lay.segments:
        t = int(g["tensor_id"])
        if not (int(g["ndim"]) == 1 and int(g["shard_stride"][0]) == 1 and int(g["canon_off"]) == 0
                and int(g["extent"][0]) == int(lay.tensors[t]["numel"])):
            return False
    return len(lay.segments) == lay.n_tensors


def _typed(lay, shards):
    import torch
    return [x.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[lay.shard_w[s]]) for s, x in enumerate(shards)]


def _choose_stage(info, avail):
    """The staging area an encode gets from `avail` bytes: every chunk's slot
    when it fits, else a compact area as large as memory allows (at least
    the plan's minimum), else none (in-order look-back)."""
    full = int(info.max_payload_bytes)
    if full <= avail:
        return full, "full"
    if int(info.compact_stage_bytes) <= avail:
        return max(int(info.compact_stage_bytes), avail // (256 << 20) * (256 << 20)), "compact"
    return 0, "in_order"


def _roof(alg_bytes, kernel_ms, traffic=None):
    a = alg_bytes / (kernel_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(a / PEAK_HBM_GBPS, 4), "traffic": traffic}


def _op_entry(name, ms_list, kms_list, alg, kalg, cb, kernel, traffic):
    ms, kms = float(np.mean(ms_list)), float(np.mean(kms_list))
    gbps = alg / (ms * 1e-3) / 1e9
    roof = _roof(kalg, kms, traffic)
    return {"ms": round(ms, 4), "alg_GB": round(alg / 1e9, 4), "alg_GBps": round(gbps, 1),
            "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4), "scanned_GBps": round(cb / (ms * 1e-3) / 1e9, 1),
            "kernel": kernel, "kernel_ms": round(kms, 4), "kernel_ms_median": round(float(np.median(kms_list)), 4),
            "kernel_alg_GB": round(kalg / 1e9, 4), "kernel_alg_GBps": roof["achieved"],
            "roofline": roof, "target_0.70": "met" if roof["frac"] >= TARGET_FRAC else "unmet"}


def _rmw_ms(recv, gbits, reps=4):
    """Best of an even number of runs of the bare read-modify-write probe
    over the groups an apply of this workload patches (the buffer ends as it
    started)."""
    import torch
    from bit_exact_xor_amd import synth
    rm = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        synth.rmw_probe_gpu(recv, gbits)
        e1.record()
        torch.cuda.synchronize()
        rm.append(e0.elapsed_time(e1))
    return min(rm)


def hot_row_share(lay, olds, news):
    """Changed elements inside the hot rows of the layout's regions, and the
    elements those rows hold."""
    import torch
    hot_changed = hot_elems = 0
    for r in lay.regions:
        if r.hot_rows is None or not r.row_len or len(r.hot_rows) == 0:
            continue
        w = lay.shard_w[r.shard]
        dt = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[w]
        o = olds[r.shard].view(dt)[r.elem_off:r.elem_off + r.n].view(-1, r.row_len)
        n = news[r.shard].view(dt)[r.elem_off:r.elem_off + r.n].view(-1, r.row_len)
        idx = torch.as_tensor(np.asarray(r.hot_rows, dtype=np.int64), device=o.device)
        hot_changed += int((o.index_select(0, idx) != n.index_select(0, idx)).sum())
        hot_elems += int(len(r.hot_rows)) * int(r.row_len)
    return hot_changed, hot_elems


def run_workload(key, make, desc, dev, args, headline=False):
    """Encode DELTA, apply, encode RETRY and retry of one workload, timed as
    `args.steps` steps after `args.warmup`; checks, per-op kernel rooflines,
    and for the headline the ceilings, the CPU baseline and the extras."""
    import torch
    from bit_exact_xor_amd import dcr, synth
    t0 = time.time()
    host_values = None
    if key == "tensor_4096x4096":
        lay = make()
        o1, n1, _lr, _pos = synth.config1_values(lay, lr=synth.CFG1_LR)
        host_values = ([o1], [n1])
    else:
        lay = make()
    T = lay.tensors
    plan = dcr.dcr_plan_build(T, [lay.shard_bytes(s) for s in range(lay.n_shards)], lay.segments)
    dcr.dcr_plan_upload(plan, dev)
    info = plan.info
    cb = int(info.canonical_bytes)
    n_chunks = int(info.n_chunks)
    log(f"{key}: plan: {info.n_tensors} tensors, {info.n_shards} shards, {n_chunks} chunks, {info.n_pieces} pieces, "
        f"{cb / 1e9:.2f} GB canonical ({time.time() - t0:.1f}s)")
    old_buf, olds = synth.alloc_shards(lay, dev)
    new_buf, news = synth.alloc_shards(lay, dev)
    if host_values is not None:
        for dst, src in zip(olds, host_values[0]):
            dst.copy_(torch.from_numpy(np.ascontiguousarray(src).view(np.uint8).reshape(-1)))
        for dst, src in zip(news, host_values[1]):
            dst.copy_(torch.from_numpy(np.ascontiguousarray(src).view(np.uint8).reshape(-1)))
    else:
        synth.fill_shards_gpu(lay, olds, 0)
        synth.fill_shards_gpu(lay, news, 1)
    torch.cuda.synchronize()

    # receiver: the canonical tensors, holding old
    if _contiguous(lay):
        recv = old_buf.clone()
        canon = _views(lay, recv, [recv[s.data_ptr() - old_buf.data_ptr():][:s.numel()] for s in olds])
        canon_new = _views(lay, new_buf, news)
    else:
        sizes = [int(T[t]["numel"]) * int(T[t]["elem_bytes"]) for t in range(len(T))]
        offs = np.concatenate([[0], np.cumsum([(s + 255) // 256 * 256 for s in sizes])]).astype(np.int64)
        recv = torch.empty(int(offs[-1]), dtype=torch.uint8, device=dev)
        canon = [recv[int(offs[t]):int(offs[t]) + sizes[t]] for t in range(len(T))]
        co = lay.assemble(_typed(lay, olds))
        for t in range(len(T)):
            canon[t].copy_(co[t].reshape(-1).view(torch.uint8))
        del co
        canon_new = [x.reshape(-1).view(torch.uint8) for x in lay.assemble(_typed(lay, news))]
    # the apply's touched 16-byte groups, 32-byte sectors and 128-byte lines,
    # and one bit per touched group of the receiver (the patch probe)
    gbits = torch.zeros((recv.numel() // 16 + 127) // 128 * 16, dtype=torch.uint8, device=dev)
    n_groups, n_sec, n_lines = _touched(canon, canon_new, gbits, [v.data_ptr() - recv.data_ptr() for v in canon])
    diff = 0
    for s in range(lay.n_shards):
        w = lay.shard_w[s]
        dt = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[w]
        diff += int((olds[s].view(dt) != news[s].view(dt)).sum())

    cap = int(cb * 0.16) + (1 << 24)
    delta = dcr.StreamBuffers(plan, dev, dir_bytes=2 * 32 * n_chunks, payload_bytes=cap)
    retry = dcr.StreamBuffers(plan, dev, dir_bytes=32 * n_chunks, payload_bytes=cap)
    flags = torch.zeros(2 * n_chunks + 1, dtype=torch.uint8, device=dev)
    ares = torch.zeros(32, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    free, _ = torch.cuda.mem_get_info()
    stage, stage_mode = _choose_stage(info, int(free) - int(info.workspace_bytes) - (3 << 30))
    ws = dcr.workspace(plan, dev, stage_bytes=stage)
    log(f"{key}: inputs, receiver and streams ready; staging {stage_mode} {stage / 1e9:.2f} GB "
        f"({time.time() - t0:.1f}s)")

    olds_t, news_t, canon_t = dcr.PtrTable(olds), dcr.PtrTable(news), dcr.PtrTable(canon)

    def encode(sb, mode):
        dcr.dcr_encode(plan, olds_t, news_t, mode, 41, 42, sb.header, sb.dir, sb.payload, sb.result, ws)

    encode(delta, 0)
    encode(retry, 1)
    torch.cuda.synchronize()
    for nm, sb in (("delta", delta), ("retry", retry)):
        r = sb.result_host()
        if int(r["status"]) != 0:
            raise SystemExit(f"{key}: {nm} stream does not fit: {r}")
    hdr, rhdr = delta.header_host(), retry.header_host()
    n_rec, p_bytes = delta.n_records(), delta.payload_bytes()
    rn_rec, rp_bytes = retry.n_records(), retry.payload_bytes()
    n_changed = int(delta.result_host()["n_changed"])

    def apply():
        flags.zero_()
        dcr.dcr_apply(plan, canon_t, hdr, delta.dir, delta.payload, flags, 0, n_rec, 41, ares, ws)

    def do_retry():
        dcr.dcr_apply_overwrite_retry(plan, canon_t, rhdr, retry.dir, retry.payload, 41, ares, ws)

    apply()
    torch.cuda.synchronize()
    ar = dcr.apply_result(ares)
    ok_apply = (int(ar["n_applied"]) == n_rec and int(ar["n_invalid"]) == 0
                and all(torch.equal(a, b) for a, b in zip(canon, canon_new)))
    do_retry()
    torch.cuda.synchronize()
    ar = dcr.apply_result(ares)
    ok_retry = (int(ar["n_applied"]) == rn_rec and int(ar["n_invalid"]) == 0
                and all(torch.equal(a, b) for a, b in zip(canon, canon_new)))
    log(f"{key}: first step: apply==new {ok_apply}, retry==new {ok_retry}; {n_rec} records {p_bytes / 1e9:.3f} GB; "
        f"retry {rn_rec} records {rp_bytes / 1e9:.3f} GB; {n_changed} changed (torch count {diff})")

    # ------------------------------------------------------------ timing
    ops = ["encode", "apply", "encode_retry", "retry"]
    fns = [lambda: encode(delta, 0), apply, lambda: encode(retry, 1), do_retry]
    for _ in range(args.warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()

    def pair():
        return (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))

    ev = [[pair() for _ in ops] for _ in range(args.steps)]      # around each call
    kev = [[pair() for _ in ops] for _ in range(args.steps)]     # around its main kernels (the library records)
    for row in kev:
        for a_, b_ in row:
            a_.record()
            b_.record()       # creates the events
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.steps):
        for i, f in enumerate(fns):
            dcr.dcr_set_kernel_events(*kev[s][i])
            ev[s][i][0].record()
            f()
            ev[s][i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    dcr.dcr_set_kernel_events(None, None)
    op_ms = {op: [ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)] for i, op in enumerate(ops)}
    kern_ms = {op: [kev[s][i][0].elapsed_time(kev[s][i][1]) for s in range(args.steps)] for i, op in enumerate(ops)}
    ms_per_step = wall * 1e3 / args.steps
    ok_after = all(torch.equal(a, b) for a, b in zip(canon, canon_new))

    # --------------------------------------------------- per-op accounting
    # the encode call reads old and new once (plus, in DELTA mode, the fp32
    # scales of block-scaled tensors once more for their routing flags) and
    # writes the records; the fix-up writes the directory.  Its tile kernels
    # read the shards and write the records.  Apply / retry read the stream
    # and every touched 128-byte line and write back every dirty 32-byte sector.
    scale_bytes = sum(int(T[int(T[t]["scale_tensor"])]["numel"]) * 4 for t in range(len(T))
                      if int(T[t]["route"]) == 2)
    alg = {"encode": 2 * cb + 2 * scale_bytes + 32 * n_rec + p_bytes,
           "apply": 32 * n_rec + p_bytes + LINE * n_lines + SECTOR * n_sec,
           "encode_retry": 2 * cb + 32 * rn_rec + rp_bytes,
           "retry": 32 * rn_rec + rp_bytes + LINE * n_lines + SECTOR * n_sec}
    kalg = {"encode": 2 * cb + p_bytes, "apply": alg["apply"], "encode_retry": 2 * cb + rp_bytes,
            "retry": alg["retry"]}
    kname = {"encode": "encode_direct_kernel", "encode_retry": "encode_direct_kernel",
             "apply": "apply_small_kernel", "retry": "apply_small_kernel"}
    per_op = {op: _op_entry(op, op_ms[op], kern_ms[op], alg[op], kalg[op], cb, kname[op],
                            measured_traffic(key, op)) for op in ops}
    rmw = _rmw_ms(recv, gbits)
    for op in ("apply", "retry"):
        per_op[op]["kernel_frac_of_rmw_ceiling"] = round(rmw / per_op[op]["kernel_ms"], 4)
    dom = max(ops, key=lambda o: sum(kern_ms[o]))
    # the dominant kernel: the op whose main kernel takes the most time per step
    roof = dict(per_op[dom]["roofline"], kernel=kname[dom], op=dom)
    value = cb / (ms_per_step * 1e-3) / 1e9
    res = {
        "workload": desc,
        "value": round(value, 2),
        "ms_per_step": round(ms_per_step, 4),
        "steps": args.steps,
        "config": {"canonical_GB": round(cb / 1e9, 3), "tensors": int(info.n_tensors),
                   "shards": int(info.n_shards), "chunks": n_chunks, "pieces": int(info.n_pieces),
                   "changed_frac": round(n_changed / sum(int(t["numel"]) for t in T), 6),
                   "step": "encode(DELTA)+apply+encode(RETRY)+retry"},
        "ops": per_op,
        "roofline": roof,
        "step_alg_GBps": round(sum(alg.values()) / (ms_per_step * 1e-3) / 1e9, 1),
        "target": {op: per_op[op]["target_0.70"] for op in ops},
        "streams": {"delta_records": n_rec, "delta_payload_GB": round(p_bytes / 1e9, 4),
                    "retry_records": rn_rec, "retry_payload_GB": round(rp_bytes / 1e9, 4),
                    "touched_16B_groups": n_groups, "touched_128B_lines": n_lines, "touched_32B_sectors": n_sec},
        "staging": {"mode": stage_mode, "stage_GB": round(stage / 1e9, 3),
                    "full_GB": round(int(info.max_payload_bytes) / 1e9, 3)},
        "rmw_ceiling_ms": round(rmw, 4),
        "checks": {"changed_eq_torch_count": n_changed == diff, "apply_eq_new": bool(ok_apply),
                   "retry_eq_new": bool(ok_retry), "after_timing_eq_new": bool(ok_after)},
    }
    log(f"{key}: {ms_per_step:.3f} ms/step, {value:.1f} GB/s scanned; " +
        ", ".join(f"{op} {per_op[op]['kernel_ms']:.3f} ms ({per_op[op]['roofline']['frac']:.3f})" for op in ops))
    if lay.meta.get("variant") == "hot":
        hc, he = hot_row_share(lay, olds, news)
        bf16 = sum(int(t["numel"]) for t in T if int(t["elem_bytes"]) == 2)
        res["hot_rows"] = {"changes_in_hot_rows": hc, "changes": n_changed,
                           "share_of_changes": round(hc / max(n_changed, 1), 4),
                           "hot_elements_frac_of_bf16": round(he / bf16, 5),
                           "note": "1% of the rows of every 2-D tensor at 100%: the largest share a 5% rate "
                                   "allows inside 1% of the rows"}

    if headline:
        res["ceiling"] = measure_ceiling(old_buf, dev, rmw=(recv, gbits, n_groups, n_lines))
        for op in ops:
            per_op[op]["kernel_frac_of_read_ceiling"] = round(
                per_op[op]["kernel_alg_GBps"] / res["ceiling"]["read_GBps"], 4)
        for op in ("apply", "retry"):   # against the bare whole-line patch of the same lines
            per_op[op]["kernel_frac_of_rmw_lines_ceiling"] = round(
                res["ceiling"]["rmw_lines"]["ms"] / per_op[op]["kernel_ms"], 4)

    # every record of both streams against the oracle, and the CPU baseline
    if headline and not args.no_cpu_baseline:
        from oracle import oracle as O
        from tests import stream_check as sc
        orc = O.get()
        streams = {0: sc.HostStream(hdr, delta.dir[:32 * n_rec].cpu().numpy(), delta.payload[:p_bytes].cpu().numpy()),
                   1: sc.HostStream(rhdr, retry.dir[:32 * rn_rec].cpu().numpy(),
                                    retry.payload[:rp_bytes].cpu().numpy())}
        lay_ok = [sc.check_layout(streams[m], lay.n_tensors, m, 41, 42, int(info.fingerprint)) for m in (0, 1)]
        cpu1, sample_ok = cpu_sample(orc, sc, lay, olds, news, streams, args.cpu_reps)
        log(f"{key}: oracle, one thread, sample: {cpu1}")
        pr = sc.full_parity(orc, lay, olds, news, streams, 41, 42, step_check=True, log=log)
        log(f"{key}: oracle over the whole workload: {pr}")
        info_h = sc.host_info()
        res["cpu_baseline"] = dict(cpu1, host=info_h, all_cores={
            "value": round(pr["canonical_bytes"] / pr["seconds"] / 1e9, 4), "unit": "GB/s",
            "cores": pr["threads"], "seconds": pr["seconds"],
            "what": "the oracle over the whole workload, one call per tensor group on a pool of threads: "
                    "encode DELTA and RETRY (every record compared with the GPU's), then the canonical old "
                    "and new tensors gathered, the DELTA stream applied and the RETRY stream retried "
                    "(result checked equal to new); value = canonical bytes / wall time"})
        res["checks"]["oracle_every_record"] = {"identical": pr["identical"], "records": pr["records"],
                                               "groups": pr["groups"], "first_mismatch": pr["first_mismatch"],
                                               "stream_layout_errors": lay_ok}
        res["checks"]["oracle_sample"] = sample_ok
        del streams

    if not args.no_extras:
        res["extras"] = workload_extras(key, lay, plan, info, olds, news, olds_t, canon, canon_t, canon_new, recv,
                                        old_buf, ws, stage, delta, retry, hdr, rhdr, n_rec, p_bytes, rn_rec,
                                        rp_bytes, flags, ares, per_op, dev)
    del ws, delta, retry, recv, canon, canon_new, gbits, old_buf, new_buf, olds, news, olds_t, news_t, canon_t
    torch.cuda.empty_cache()
    return res


def cpu_sample(orc, sc, lay, olds, news, streams, reps):
    """The oracle on one thread over a bounded sample of the workload: layer
    0's attention, norm and router tensors and its experts 0..31 (with their
    scale tensors).  One step = encode DELTA + encode RETRY + apply + retry;
    the gather of the receiver's canonical old tensors is setup, not timed.
    Also compares the sample's records with the GPU streams."""
    names = lay.tensor_names
    ids = []
    for i, n in enumerate(names):
        if not n.startswith("model.layers.0."):
            continue
        if ".mlp.experts." in n:
            e = int(n.split(".mlp.experts.")[1].split(".")[0])
            if e >= 32:
                continue
        ids.append(i)
    ids = sorted(ids)
    T, S, so, sn = sc.mini_inputs(lay, ids, olds, news)
    sample_bytes = int(sum(int(t["numel"]) * int(t["elem_bytes"]) for t in T))
    times = []
    same = None
    for rep in range(reps):
        t0 = time.perf_counter()
        if rep == 0:
            outs = {}
            _n, _b, err = sc._compare_group(orc, ids, T, S, so, sn, streams, 41, 42, 0, outs)
            same = err is None
            (h, d, p), (rh, rd, rp) = outs[0], outs[1]
        else:
            rc, h, d, p = orc.encode(T, S, so, sn, mode=0, base_version=41, new_version=42,
                                     dir_cap=len(outs[0][1]), payload_cap=len(outs[0][2]))
            rc2, rh, rd, rp = orc.encode(T, S, so, sn, mode=1, base_version=41, new_version=42,
                                         dir_cap=len(outs[1][1]), payload_cap=len(outs[1][2]))
            assert rc == 0 and rc2 == 0
        t1 = time.perf_counter()
        canon = [orc.gather(T, S, so, t) for t in range(len(T))]
        t2 = time.perf_counter()
        f = np.zeros(max(len(d) // 32, 1), np.uint8)
        assert orc.apply(T, canon, h, d, p, f, expected_base_version=41) == 0
        assert orc.retry(T, canon, rh, rd, rp, expected_base_version=41) == 0
        t3 = time.perf_counter()
        times.append((t1 - t0) + (t3 - t2))
    step_s = float(np.median(times))
    return ({"value": round(sample_bytes / step_s / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
             "sample": f"layer 0 of the same workload: attention, norms, router and experts 0..31 with their "
                       f"scale tensors ({len(T)} tensors, {sample_bytes / 1e6:.1f} MB); one step = encode DELTA "
                       f"+ encode RETRY + apply + retry; median of {reps}",
             "step_s": round(step_s, 3)},
            {"tensors": len(T), "identical": bool(same)})


def workload_extras(key, lay, plan, info, olds, news, olds_t, canon, canon_t, canon_new, recv, old_buf, ws, stage,
                    delta, retry, hdr, rhdr, n_rec, p_bytes, rn_rec, rp_bytes, flags, ares, per_op, dev):
    """Measurements outside the step, each with its own check.  Every
    workload: the RETRY stream written from the DELTA stream.  The Llama-8B
    workload also: partial retry, index lists, a TP=2 receiver layout, the
    pipelined transfer and the staging-area sizes.  The small tensor: a
    HIP-graph replay of encode + apply."""
    import torch
    from bit_exact_xor_amd import dcr, synth
    T = lay.tensors
    ex = {}
    contiguous = _contiguous(lay)

    def reset_old():
        if contiguous:
            recv.copy_(old_buf)
        else:
            co = lay.assemble(_typed(lay, olds))
            for t in range(len(T)):
                canon[t].copy_(co[t].reshape(-1).view(torch.uint8))
            del co

    def eq_new():
        return all(torch.equal(a, b) for a, b in zip(canon, canon_new))

    def pair():
        return (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))

    def timed3(fn, reps=3):
        ts = []
        for _ in range(reps):
            a_, b_ = pair()
            a_.record()
            fn()
            b_.record()
            torch.cuda.synchronize()
            ts.append(a_.elapsed_time(b_))
        return round(float(np.median(ts)), 4)

    # the RETRY stream written from the DELTA stream and old only, into fresh
    # buffers filled with a poison byte; compared byte for byte with the
    # RETRY encode's stream, then applied to old, which must give new
    tsb = dcr.StreamBuffers(plan, dev, dir_bytes=32 * int(info.n_chunks), payload_bytes=rp_bytes + (1 << 20))
    tsb.header.fill_(0xA5)
    tsb.dir.fill_(0xA5)
    tsb.payload.fill_(0xA5)
    ms = timed3(lambda: dcr.dcr_encode_retry_from_delta(plan, olds_t, hdr, delta.dir, delta.payload, 0, tsb.header,
                                                         tsb.dir, tsb.payload, tsb.result, ws))
    tr = tsb.result_host()
    same = (int(tr["status"]) == 0 and int(tr["n_records"]) == rn_rec and int(tr["payload_bytes"]) == rp_bytes
            and torch.equal(tsb.header, retry.header) and torch.equal(tsb.dir[:32 * rn_rec], retry.dir[:32 * rn_rec])
            and torch.equal(tsb.payload[:rp_bytes], retry.payload[:rp_bytes]))
    reset_old()
    dcr.dcr_apply_overwrite_retry(plan, canon_t, tsb.header_host(), tsb.dir, tsb.payload, 41, ares, ws)
    torch.cuda.synchronize()
    ex["retry_from_delta"] = {"ms": ms, "retry_encode_ms": per_op["encode_retry"]["ms"],
                              "stream_eq_retry_encode": bool(same), "applied_to_old_eq_new": bool(eq_new())}
    del tsb
    log(f"{key}: RETRY stream from the DELTA stream: {ex['retry_from_delta']}")

    if key == "tensor_4096x4096":
        # launch-bound: encode (staged) + apply captured once in a HIP graph
        # and replayed, against the same calls eager
        gsb = dcr.StreamBuffers(plan, dev, dir_bytes=2 * 32 * int(info.n_chunks), payload_bytes=p_bytes + (1 << 20))
        wsg = dcr.workspace(plan, dev, stage)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            dcr.dcr_encode(plan, olds_t, dcr.PtrTable(news), 0, 41, 42, gsb.header, gsb.dir, gsb.payload,
                           gsb.result, wsg)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        news_t = dcr.PtrTable(news)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            dcr.dcr_encode(plan, olds_t, news_t, 0, 41, 42, gsb.header, gsb.dir, gsb.payload, gsb.result, wsg)
            flags.zero_()
            dcr.dcr_apply(plan, canon_t, hdr, gsb.dir, gsb.payload, flags, 0, n_rec, 41, ares, ws)
        gsb.dir.fill_(0xEE)
        g.replay()
        torch.cuda.synchronize()
        same = (torch.equal(gsb.header, delta.header) and torch.equal(gsb.dir[:32 * n_rec], delta.dir[:32 * n_rec])
                and torch.equal(gsb.payload[:p_bytes], delta.payload[:p_bytes]))
        gt, et = [], []
        for _ in range(20):
            a_, b_ = pair()
            a_.record()
            g.replay()
            b_.record()
            torch.cuda.synchronize()
            gt.append(a_.elapsed_time(b_))
            a_, b_ = pair()
            a_.record()
            dcr.dcr_encode(plan, olds_t, news_t, 0, 41, 42, delta.header, delta.dir, delta.payload, delta.result, ws)
            flags.zero_()
            dcr.dcr_apply(plan, canon_t, hdr, delta.dir, delta.payload, flags, 0, n_rec, 41, ares, ws)
            b_.record()
            torch.cuda.synchronize()
            et.append(a_.elapsed_time(b_))
        ex["graph"] = {"encode_apply_replay_ms": round(float(np.median(gt)), 4),
                       "encode_apply_eager_ms": round(float(np.median(et)), 4), "stream_eq_eager": bool(same)}
        del g, gsb, wsg
        log(f"{key}: graph replay: {ex['graph']}")

    if key != "llama8b_tp4":
        return ex

    # partial retry after a kill at 50 % of the DELTA records: the receiver
    # is set back to old, applies the first half, and the sender re-encodes
    # only the chunks of the unflagged records
    reset_old()
    flags.zero_()
    dcr.dcr_apply(plan, canon_t, hdr, delta.dir, delta.payload, flags, 0, n_rec // 2, 41, ares, ws)
    torch.cuda.synchronize()
    psb = dcr.StreamBuffers(plan, dev, dir_bytes=32 * int(info.n_chunks), payload_bytes=rp_bytes + (1 << 20))
    pe = timed3(lambda: dcr.dcr_encode_retry_partial(plan, olds_t, dcr.PtrTable(news), hdr, delta.dir, flags, 41,
                                                     42, psb.header, psb.dir, psb.payload, psb.result, ws))
    pr, ph = psb.result_host(), psb.header_host()
    pa = timed3(lambda: dcr.dcr_apply_overwrite_retry(plan, canon_t, ph, psb.dir, psb.payload, 41, ares, ws))
    ex["partial_retry"] = {"kill_at_records": n_rec // 2, "status": int(pr["status"]), "records": int(pr["n_records"]),
                           "payload_GB": round(int(pr["payload_bytes"]) / 1e9, 4),
                           "full_retry_payload_GB": round(rp_bytes / 1e9, 4), "encode_ms": pe,
                           "full_retry_encode_ms": per_op["encode_retry"]["ms"], "apply_ms": pa,
                           "full_retry_apply_ms": per_op["retry"]["ms"], "healed_eq_new": bool(eq_new())}
    del psb
    log(f"{key}: partial retry at a 50 % kill: {ex['partial_retry']}")

    # index-list layout (encode option): the same DELTA change set with
    # low-density records carrying 16-bit indices instead of the bitmap
    lsb = dcr.StreamBuffers(plan, dev, dir_bytes=2 * 32 * int(info.n_chunks), payload_bytes=p_bytes + (1 << 20))
    le = timed3(lambda: dcr.dcr_encode(plan, olds_t, dcr.PtrTable(news), dcr.MODE_DELTA | dcr.ENC_INDEX_LISTS, 41,
                                       42, lsb.header, lsb.dir, lsb.payload, lsb.result, ws))
    lr, lh = lsb.result_host(), lsb.header_host()
    ln = int(lr["n_records"])
    lflags = torch.zeros(max(ln, 1), dtype=torch.uint8, device=dev)
    la = []
    for _ in range(3):
        reset_old()
        lflags.zero_()
        torch.cuda.synchronize()
        a_, b_ = pair()
        a_.record()
        dcr.dcr_apply(plan, canon_t, lh, lsb.dir, lsb.payload, lflags, 0, ln, 41, ares, ws)
        b_.record()
        torch.cuda.synchronize()
        la.append(a_.elapsed_time(b_))
    ex["index_lists"] = {"status": int(lr["status"]), "records": ln,
                         "payload_GB": round(int(lr["payload_bytes"]) / 1e9, 4),
                         "bitmap_payload_GB": round(p_bytes / 1e9, 4), "encode_ms": le,
                         "bitmap_encode_ms": per_op["encode"]["ms"], "apply_ms": round(float(np.median(la)), 4),
                         "bitmap_apply_ms": per_op["apply"]["ms"], "apply_eq_new": bool(eq_new())}
    del lsb, lflags
    log(f"{key}: index-list layout: {ex['index_lists']}")

    # apply straight into receivers that store the model in their own
    # layout: TP=2 engine shards; TP=4 engine shards whose fused gate/up
    # weight interleaves gate and up rows in groups of 64
    for rname, lay_r, what in (
            ("sharded_apply", synth.llama_layout(tp=2), "the same model as TP=2 engine shards"),
            ("sharded_apply_gate_up64", synth.llama_layout(tp=4, gate_up_group=64),
             "TP=4 engine shards, fused gate/up rows interleaved in groups of 64")):
        rplan = dcr.dcr_plan_build(lay_r.tensors, [lay_r.shard_bytes(s) for s in range(lay_r.n_shards)],
                                   lay_r.segments)
        dcr.dcr_plan_upload(rplan, dev)
        rws = dcr.workspace(rplan, dev)
        canon_o = lay.assemble(_typed(lay, olds))
        rbuf, rsh = synth.scatter_canonical_gpu(lay_r, canon_o, dev)
        del canon_o
        torch.cuda.synchronize()
        sa = []
        for _ in range(3):       # XOR records toggle old -> new -> old -> new
            flags.zero_()
            a_, b_ = pair()
            a_.record()
            dcr.dcr_apply_sharded(rplan, rsh, hdr, delta.dir, delta.payload, flags, 0, n_rec, 41, ares, rws)
            b_.record()
            torch.cuda.synchronize()
            sa.append(a_.elapsed_time(b_))
        got = lay_r.assemble(_typed(lay_r, rsh))
        ok_sharded = all(torch.equal(got[t].reshape(-1).view(torch.uint8), canon_new[t]) for t in range(len(T)))
        del got, rbuf, rsh, rws
        torch.cuda.empty_cache()
        ex[rname] = {"receiver": f"{what} ({rplan.info.n_shards} shards, {rplan.info.n_pieces} pieces)",
                     "apply_ms": round(float(np.median(sa)), 4), "canonical_apply_ms": per_op["apply"]["ms"],
                     "eq_new": bool(ok_sharded)}
        log(f"{key}: apply into a receiver layout: {ex[rname]}")

    ex["pipelined"] = pipelined_transfer(plan, lay, olds, news, canon, lambda v: _typed(lay, v), ws, delta, n_rec,
                                         p_bytes, dev, per_op["encode"]["ms"], per_op["apply"]["ms"])
    log(f"{key}: pipelined transfer through pinned host memory: {ex['pipelined']}")

    # staging area sizes: the whole worst case, compact areas of 4 GiB,
    # 2 GiB and the plan's minimum, and none (in-order look-back); each
    # stream compared with the step's
    sm = {"compact_stage_bytes": int(info.compact_stage_bytes), "full_stage_bytes": int(info.max_payload_bytes)}
    ref = (delta.header.clone(), delta.dir[:32 * n_rec].clone(), delta.payload[:p_bytes].clone())
    news_t = dcr.PtrTable(news)
    for name, sbytes in (("full", int(info.max_payload_bytes)), ("compact_4GiB", 4 << 30),
                         ("compact_2GiB", 2 << 30), ("compact_min", int(info.compact_stage_bytes)), ("in_order", 0)):
        wsm = dcr.workspace(plan, dev, stage_bytes=sbytes)
        tm = []
        for _ in range(4):
            a_, b_ = pair()
            a_.record()
            dcr.dcr_encode(plan, olds_t, news_t, 0, 41, 42, delta.header, delta.dir, delta.payload, delta.result, wsm)
            b_.record()
            torch.cuda.synchronize()
            tm.append(a_.elapsed_time(b_))
        same = (torch.equal(delta.header, ref[0]) and torch.equal(delta.dir[:32 * n_rec], ref[1])
                and torch.equal(delta.payload[:p_bytes], ref[2]))
        sm[name] = {"stage_GB": round(sbytes / 1e9, 3), "encode_ms": round(float(np.median(tm[1:])), 3),
                    "reencoded_chunks": int(delta.result_host()["n_reencoded"]),
                    "stream_eq": bool(same)}
        del wsm
        torch.cuda.empty_cache()
    ex["staging_modes"] = sm
    del ref
    log(f"{key}: staging area sizes: {sm}")
    return ex


def run_receiver_share(desc, dev, args, window=256):
    """The 240 GB receiver share: streams built window by window (the new
    values never fit beside the receiver), then the DELTA apply of every
    record and the overwrite retry of every record, each timed over
    `args.steps` runs in place.  The two streams are not resident together
    (240 GB of receiver state leaves room for one): the step time is the sum
    of the two ops' mean times."""
    import torch
    from bit_exact_xor_amd import dcr, synth
    from tests import stream_check as sc
    t0 = time.time()
    lay = synth.config5_layout()
    T = lay.tensors
    plan_full = dcr.dcr_plan_build(T, [lay.shard_bytes(s) for s in range(lay.n_shards)], lay.segments)
    dcr.dcr_plan_upload(plan_full, dev)
    n_chunks = int(plan_full.info.n_chunks)
    free, _ = torch.cuda.mem_get_info()
    need = 240 * 10**9 + 2 * 8 * 10**9 + 28 * 10**9 + 2 * 10**9
    if free < need:
        return {"workload": desc, "skipped": f"needs {need / 1e9:.0f} GB of free HBM, {free / 1e9:.0f} GB available"}
    sizes = [lay.shard_bytes(s) for s in range(lay.n_shards)]
    offs = np.concatenate([[0], np.cumsum([(s + 255) // 256 * 256 for s in sizes])]).astype(np.int64)
    cbuf = torch.empty(int(offs[-1]), dtype=torch.uint8, device=dev)
    canon = [cbuf[int(offs[t]):int(offs[t]) + sizes[t]] for t in range(len(sizes))]
    synth.fill_shards_gpu(lay, canon, 0)
    wbytes = max(sum((sizes[t] + 255) // 256 * 256 for t in range(a, min(len(sizes), a + window)))
                 for a in range(0, len(sizes), window))
    t_old = torch.empty(wbytes, dtype=torch.uint8, device=dev)
    t_new = torch.empty(wbytes, dtype=torch.uint8, device=dev)
    gbits = torch.zeros((cbuf.numel() // 16 + 127) // 128 * 16, dtype=torch.uint8, device=dev)
    ws = dcr.workspace(plan_full, dev)
    res = torch.zeros(32, dtype=torch.uint8, device=dev)
    touched = [0, 0, 0]

    def build(mode, dir_buf, payload, count):
        r_off = p_off = changed = 0
        for a in range(0, lay.n_tensors, window):
            b_ = min(lay.n_tensors, a + window)
            wl = synth.window_layout(lay, a, b_)
            plan = dcr.dcr_plan_build(wl.tensors, [wl.shard_bytes(s) for s in range(wl.n_shards)], wl.segments)
            dcr.dcr_plan_upload(plan, dev)
            olds, news, off = [], [], 0
            for s in range(wl.n_shards):
                nb = wl.shard_bytes(s)
                olds.append(t_old[off:off + nb])
                news.append(t_new[off:off + nb])
                off += (nb + 255) // 256 * 256
            synth.fill_shards_gpu(wl, olds, 0)
            synth.fill_shards_gpu(wl, news, 1)
            if count:
                gi, si, li = _touched(olds, news, gbits,
                                      [canon[a + i].data_ptr() - cbuf.data_ptr() for i in range(b_ - a)])
                touched[0] += gi
                touched[1] += si
                touched[2] += li
            wsw = dcr.workspace(plan, dev)
            hdr_w = torch.zeros(64, dtype=torch.uint8, device=dev)
            rs = torch.zeros(32, dtype=torch.uint8, device=dev)
            dcr.dcr_encode(plan, olds, news, mode, 5, 6, hdr_w, dir_buf[r_off * 32:], payload[p_off:], rs, wsw)
            torch.cuda.synchronize()
            r = np.frombuffer(rs.cpu().numpy().tobytes(), dtype=dcr.ENCODE_RESULT)[0]
            assert int(r["status"]) == 0, (a, r)
            n, pb = int(r["n_records"]), int(r["payload_bytes"])
            if n:
                e32 = dir_buf[r_off * 32:(r_off + n) * 32].view(torch.int32).view(-1, 8)
                e64 = dir_buf[r_off * 32:(r_off + n) * 32].view(torch.int64).view(-1, 4)
                e32[:, 0] += a
                e64[:, 2] += p_off
            r_off += n
            p_off += pb
            changed += int(r["n_changed"])
        hdr = np.zeros(64, dtype=np.uint8)
        h = hdr.view(np.uint32)
        h[0], h[2] = 0x31524344, 65536
        hdr[4:6].view(np.uint16)[0] = 1
        hdr[6:8].view(np.uint16)[0] = mode
        hdr[16:24].view(np.uint64)[0] = 5
        hdr[24:32].view(np.uint64)[0] = 6
        hdr[32:40].view(np.uint64)[0] = plan_full.info.fingerprint
        hdr[40:48].view(np.uint64)[0] = r_off
        hdr[48:56].view(np.uint64)[0] = p_off
        hs = sc.HostStream(hdr, dir_buf[:32 * r_off].cpu().numpy(), None, p_len=p_off)
        err = sc.check_layout(hs, lay.n_tensors, mode, 5, 6, int(plan_full.info.fingerprint))
        assert err is None, err
        return hdr, r_off, p_off, changed

    def eq_new():
        ok = True
        for a in range(0, lay.n_tensors, window):
            b_ = min(lay.n_tensors, a + window)
            wl = synth.window_layout(lay, a, b_)
            news, off = [], 0
            for s in range(wl.n_shards):
                nb = wl.shard_bytes(s)
                news.append(t_new[off:off + nb])
                off += (nb + 255) // 256 * 256
            synth.fill_shards_gpu(wl, news, 1)
            ok = ok and all(torch.equal(canon[a + i], news[i]) for i in range(b_ - a))
        return ok

    cb = int(plan_full.info.canonical_bytes)
    dir_buf = torch.empty(32 * n_chunks, dtype=torch.uint8, device=dev)
    payload = torch.empty(26 * 10**9, dtype=torch.uint8, device=dev)
    hdr, n_rec, p_bytes, changed = build(0, dir_buf, payload, True)
    log(f"receiver share: DELTA stream {n_rec} records, {p_bytes / 1e9:.2f} GB ({time.time() - t0:.0f}s)")
    flags = torch.zeros(n_rec, dtype=torch.uint8, device=dev)
    canon_t = dcr.PtrTable(canon)

    def apply():
        flags.zero_()
        dcr.dcr_apply(plan_full, canon_t, hdr, dir_buf, payload, flags, 0, n_rec, 5, res, ws)

    # every run applies the same XOR stream: old -> new -> old ...; an odd
    # count of runs ends at new
    n_a = args.steps if args.steps % 2 else args.steps + 1
    a_ms, a_kms = _timed(apply, n_a)
    ar = dcr.apply_result(res)
    ok_apply = int(ar["n_applied"]) == n_rec and int(ar["n_invalid"]) == 0 and eq_new()
    rmw = _rmw_ms(cbuf, gbits)
    del dir_buf, payload, flags
    torch.cuda.empty_cache()
    rdir = torch.empty(32 * n_chunks, dtype=torch.uint8, device=dev)
    rpay = torch.empty(28 * 10**9, dtype=torch.uint8, device=dev)
    rhdr, rn, rpb, _ = build(1, rdir, rpay, False)
    log(f"receiver share: RETRY stream {rn} records, {rpb / 1e9:.2f} GB ({time.time() - t0:.0f}s)")
    t_ms, t_kms = _timed(lambda: dcr.dcr_apply_overwrite_retry(plan_full, canon_t, rhdr, rdir, rpay, 5, res, ws),
                         args.steps)
    ar = dcr.apply_result(res)
    ok_retry = int(ar["n_applied"]) == rn and int(ar["n_invalid"]) == 0 and eq_new()
    g, s_, l_ = touched
    a_alg = 32 * n_rec + p_bytes + LINE * l_ + SECTOR * s_
    r_alg = 32 * rn + rpb + LINE * l_ + SECTOR * s_
    ops = {"apply": _op_entry("apply", a_ms, a_kms, a_alg, a_alg, cb, "apply_small_kernel",
                              measured_traffic("receiver_share_240GB", "apply")),
           "retry": _op_entry("retry", t_ms, t_kms, r_alg, r_alg, cb, "apply_small_kernel",
                              measured_traffic("receiver_share_240GB", "retry"))}
    for op in ops:
        ops[op]["kernel_frac_of_rmw_ceiling"] = round(rmw / ops[op]["kernel_ms"], 4)
    ms_step = ops["apply"]["ms"] + ops["retry"]["ms"]
    dom = max(ops, key=lambda o: ops[o]["kernel_ms"])
    out = {"workload": desc, "value": round(cb / (ms_step * 1e-3) / 1e9, 2), "ms_per_step": round(ms_step, 4),
           "steps": args.steps,
           "config": {"canonical_GB": round(cb / 1e9, 3), "tensors": int(plan_full.info.n_tensors),
                      "chunks": n_chunks, "changed": changed, "step": "apply + retry (mean op times)"},
           "ops": ops, "roofline": dict(ops[dom]["roofline"], kernel="apply_small_kernel", op=dom),
           "target": {op: ops[op]["target_0.70"] for op in ops},
           "streams": {"delta_records": n_rec, "delta_payload_GB": round(p_bytes / 1e9, 4),
                       "retry_records": rn, "retry_payload_GB": round(rpb / 1e9, 4),
                       "touched_16B_groups": g, "touched_128B_lines": l_, "touched_32B_sectors": s_},
           "rmw_ceiling_ms": round(rmw, 4),
           "checks": {"apply_eq_new": bool(ok_apply), "retry_eq_new": bool(ok_retry),
                      "oracle_every_record": "in the GPU tests (window by window); not repeated here"},
           "note": "apply-only workload: the streams are built window by window outside the timing"}
    del cbuf, canon, canon_t, rdir, rpay, t_old, t_new, gbits, ws
    torch.cuda.empty_cache()
    return out



def pipelined_transfer(plan, lay, olds, news, canon, as_i16, ws, sb, n_rec, p_bytes, dev, encode_ms, apply_ms,
                       n_slices=16, reps=5):
    """Latency of moving a refit through pinned host memory (PCIe both ways;
    the host buffer stands in for the network), without and with pipelining
    (outside the step; the receiver is reset to old before each run):
      sender    first encoded byte to the whole stream in host memory: the
                encode then one copy out, against the pipelined encode whose
                published slices are copied out while it runs;
      receiver  stream in host memory to the last patched weight: one copy in
                then one apply, against per-slice copies double-buffered
                against per-slice applies;
      loopback  both on this one GPU, which share its PCIe link and copy
                engines (two machines would not)."""
    import torch
    from bit_exact_xor_amd import dcr
    from bit_exact_xor_amd.pipeline import HostLoopback
    T = lay.tensors
    canon_o = lay.assemble(as_i16(olds))
    canon_new = lay.assemble(as_i16(news))
    lb = HostLoopback(plan, 32 * n_rec + (1 << 16), p_bytes + (1 << 20), dev)
    rws = dcr.workspace(plan, dev)
    flags = torch.zeros(max(n_rec, 1), dtype=torch.uint8, device=dev)

    def reset():
        for t in range(len(T)):
            canon[t].view(torch.int16).copy_(canon_o[t].reshape(-1))
        flags.zero_()
        torch.cuda.synchronize()

    def eq_new():
        return all(torch.equal(canon[t].view(torch.int16), canon_new[t].reshape(-1)) for t in range(len(T)))

    def timed(f):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        r = f()
        torch.cuda.synchronize()
        return time.perf_counter() - t0, r

    # PCIe rates of the payload alone, for reference
    d2h, h2d = [], []
    for _ in range(3):
        d2h.append(timed(lambda: lb.host_payload[:p_bytes].copy_(sb.payload[:p_bytes], non_blocking=True))[0])
        h2d.append(timed(lambda: lb.rpayload[:p_bytes].copy_(lb.host_payload[:p_bytes], non_blocking=True))[0])
    # the sliced encode alone (slices published, nothing copied)
    sl = []
    ready = torch.zeros(dcr.ready_region_bytes(n_slices), dtype=torch.uint8, pin_memory=True)
    for _ in range(reps):
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a_.record()
        dcr.dcr_encode_pipelined(plan, olds, news, 0, 41, 42, sb.header, sb.dir, sb.payload, sb.result, ws,
                                 n_slices, ready)
        b_.record()
        torch.cuda.synchronize()
        sl.append(a_.elapsed_time(b_))
    res = {k: [] for k in ("send_serial", "send_pipelined", "recv_serial", "recv_pipelined", "loop_serial",
                           "loop_pipelined")}
    ok = {"sender_stream": True, "recv_serial": True, "recv_pipelined": True, "loop_serial": True,
          "loop_pipelined": True}
    ref_dir, ref_pay = sb.dir[: 32 * n_rec].cpu(), sb.payload[:p_bytes].cpu()
    heads = None
    for _ in range(reps):
        dt, hdr = timed(lambda: lb.send_serial(olds, news, 0, 41, 42, sb, ws))
        res["send_serial"].append(dt)
        dt, (heads, _) = timed(lambda: lb.send(olds, news, 0, 41, 42, sb, ws, n_slices))
        res["send_pipelined"].append(dt)
        ok["sender_stream"] &= bool(torch.equal(lb.host_dir[: 32 * n_rec], ref_dir) and
                                    torch.equal(lb.host_payload[:p_bytes], ref_pay))
        reset()
        res["recv_serial"].append(timed(lambda: lb.receive_serial(hdr, canon, flags, rws, 41))[0])
        ok["recv_serial"] &= eq_new()
        reset()
        res["recv_pipelined"].append(timed(lambda: lb.receive(heads, canon, flags, rws, 41))[0])
        ok["recv_pipelined"] &= eq_new()
        reset()
        res["loop_serial"].append(timed(lambda: lb.run_serial(olds, news, 0, 41, 42, sb, ws, canon, flags, rws))[0])
        ok["loop_serial"] &= eq_new()
        reset()
        res["loop_pipelined"].append(timed(lambda: lb.run(olds, news, 0, 41, 42, sb, ws, n_slices, canon, flags,
                                                          rws))[0])
        ok["loop_pipelined"] &= eq_new()
    del canon_o, canon_new, lb, rws
    torch.cuda.empty_cache()
    med = {k: round(float(np.median(v)) * 1e3, 3) for k, v in res.items()}
    out = {"slices": len(heads), "payload_GB": round(p_bytes / 1e9, 4),
           "d2h_GBps": round(p_bytes / float(np.median(d2h)) / 1e9, 1),
           "h2d_GBps": round(p_bytes / float(np.median(h2d)) / 1e9, 1),
           "encode_ms": round(encode_ms, 3), "encode_sliced_ms": round(float(np.median(sl)), 3),
           "apply_ms": round(apply_ms, 3), "median_ms": med,
           "loop_pipelined_min_ms": round(min(res["loop_pipelined"]) * 1e3, 3),
           "speedup": {k: round(med[k + "_serial"] / med[k + "_pipelined"], 3) for k in ("send", "recv", "loop")},
           "checks": ok}
    return out


def _pack_roundtrip(plan, sb, hdr, n, pb, ws, dev, reps):
    """The transport packing of a finished stream and back: packed payload
    bytes, records by layout (bitmap / list / gap varints), pack and unpack
    times (median of reps) and the unpacked stream compared with the
    original byte for byte (its payload buffer poisoned first)."""
    import torch
    from bit_exact_xor_amd import dcr
    ps = dcr.StreamBuffers(plan, dev, dir_bytes=32 * max(n, 1), payload_bytes=max(pb, 16))
    us = dcr.StreamBuffers(plan, dev, dir_bytes=32 * max(n, 1), payload_bytes=max(pb, 16))
    us.payload.fill_(0xA5)
    t = {"pack": [], "unpack": []}
    for op in ("pack", "unpack"):
        for _ in range(reps):
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record()
            if op == "pack":
                dcr.dcr_stream_pack(plan, hdr, sb.dir, sb.payload, ps.header, ps.dir, ps.payload, ps.result, ws)
            else:
                dcr.dcr_stream_unpack(plan, ps.header.cpu().numpy(), ps.dir, ps.payload, us.header, us.dir,
                                      us.payload, us.result, ws)
            b_.record()
            torch.cuda.synchronize()
            t[op].append(a_.elapsed_time(b_))
    pr, ur = ps.result_host(), us.result_host()
    ppb = int(pr["payload_bytes"])
    layouts = np.bincount(ps.dir[: 32 * n].view(-1, 32)[:, 15].cpu().numpy(), minlength=3) if n else [0, 0, 0]
    same = (int(pr["status"]) == 0 and int(ur["status"]) == 0 and int(ur["payload_bytes"]) == pb
            and torch.equal(us.header, sb.header) and torch.equal(us.dir[: 32 * n], sb.dir[: 32 * n])
            and torch.equal(us.payload[:pb], sb.payload[:pb]))
    return {"payload_GB": round(ppb / 1e9, 4), "records_by_layout": [int(x) for x in layouts[:3]],
            "pack_ms": round(float(np.median(t["pack"])), 3), "unpack_ms": round(float(np.median(t["unpack"])), 3),
            "unpacked_eq_stream": bool(same)}


def lists_cfg5(dev, reps=3):
    """Bitmap against index-list streams on config 5's two regions (identity
    layouts: shard i = tensor i, so the old shards are the canonical old
    tensors): stream bytes, encode and apply times (median of reps), the
    weights after an odd number of XOR applies checked against new, and the
    index-list stream's transport packing and back."""
    import torch
    from bit_exact_xor_amd import dcr, synth
    out = {}
    for name, kw in (("nvfp4 uint8, 0.085 % of bytes", dict(n_bf16=0, n_u8=5450)),
                     ("bf16, 3 % (1000 of the 6812 tensors)", dict(n_bf16=1000, n_u8=0))):
        lay = synth.config5_layout(**kw)
        plan = dcr.dcr_plan_build(lay.tensors, [lay.shard_bytes(s) for s in range(lay.n_shards)], lay.segments)
        dcr.dcr_plan_upload(plan, dev)
        ob, olds = synth.alloc_shards(lay, dev)
        nb, news = synth.alloc_shards(lay, dev)
        synth.fill_shards_gpu(lay, olds, 0)
        synth.fill_shards_gpu(lay, news, 1)
        cb = int(plan.info.canonical_bytes)
        cbuf = ob.clone()
        canon = [cbuf[int(o.data_ptr() - ob.data_ptr()):int(o.data_ptr() - ob.data_ptr()) + o.numel()] for o in olds]
        ws = dcr.workspace(plan, dev, int(plan.info.max_payload_bytes))
        sb = dcr.StreamBuffers(plan, dev, dir_bytes=2 * 32 * int(plan.info.n_chunks),
                               payload_bytes=int(cb * 0.2) + (1 << 20))
        res = torch.zeros(32, dtype=torch.uint8, device=dev)
        row = {}
        for lname, opt in (("bitmap", 0), ("lists", dcr.ENC_INDEX_LISTS)):
            te, ta = [], []
            for _ in range(reps):
                a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a_.record()
                dcr.dcr_encode(plan, olds, news, dcr.MODE_DELTA | opt, 1, 2, sb.header, sb.dir, sb.payload,
                               sb.result, ws)
                b_.record()
                torch.cuda.synchronize()
                te.append(a_.elapsed_time(b_))
            r = sb.result_host()
            n = int(r["n_records"])
            hdr = sb.header_host()
            flags = torch.zeros(max(n, 1), dtype=torch.uint8, device=dev)
            cbuf.copy_(ob)
            for _ in range(reps):          # XOR records toggle old -> new -> old -> new
                flags.zero_()
                a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a_.record()
                dcr.dcr_apply(plan, canon, hdr, sb.dir, sb.payload, flags, 0, n, 1, res, ws)
                b_.record()
                torch.cuda.synchronize()
                ta.append(a_.elapsed_time(b_))
            row[lname] = {"status": int(r["status"]), "records": n,
                          "payload_GB": round(int(r["payload_bytes"]) / 1e9, 4),
                          "encode_ms": round(float(np.median(te)), 3), "apply_ms": round(float(np.median(ta)), 3),
                          "apply_eq_new": all(torch.equal(c, x) for c, x in zip(canon, news))}
            if opt:
                row[lname]["packed"] = _pack_roundtrip(plan, sb, hdr, n, int(r["payload_bytes"]), ws, dev, reps)
        out[name] = {"canonical_GB": round(cb / 1e9, 3), **row}
        log(f"{name}: {out[name]}")
        del ob, nb, olds, news, cbuf, canon, ws, sb, plan
        torch.cuda.empty_cache()
    return {"lists_cfg5": out}


def _views(lay, buf, shards):
    """Per canonical tensor, a view of the flat shard buffer holding it (every
    tensor of these layouts is one contiguous run of one shard)."""
    import torch
    base = buf.data_ptr()
    out = [None] * lay.n_tensors
    for g in lay.segments:
        t, sh = int(g["tensor_id"]), int(g["shard_id"])
        n, w = int(lay.tensors[t]["numel"]), int(lay.tensors[t]["elem_bytes"])
        assert int(g["ndim"]) == 1 and int(g["shard_stride"][0]) == 1 and int(g["canon_off"]) == 0
        assert int(g["extent"][0]) == n and out[t] is None
        o = shards[sh].data_ptr() - base + int(g["shard_off"]) * w
        out[t] = buf[o:o + n * w]
    return out


def _touched(old_views, new_views, gbits_buf, byte_offs):
    """Touched 16-byte groups, 32-byte sectors and 128-byte lines of the
    tensors (old vs new bytes); sets each touched group's bit in gbits_buf,
    one bit per 16-byte group of the flat receiver buffer in which tensor i
    starts at byte byte_offs[i] (a multiple of 128)."""
    import torch
    g = s_ = l_ = 0
    for o, n, boff in zip(old_views, new_views, byte_offs):
        nb = o.numel()
        assert nb % 16 == 0 and boff % 128 == 0
        d = (o.view(torch.int64) != n.view(torch.int64)).view(-1, 2).any(1)
        ng = d.numel()
        g += int(d.sum())
        pad = torch.zeros((ng + 7) // 8 * 8, dtype=torch.bool, device=d.device)
        pad[:ng] = d
        sec = pad.view(-1, 2).any(1)
        s_ += int(sec.sum())
        l_ += int(pad.view(-1, 8).any(1).sum())
        g0 = boff // 16
        byte = torch.zeros(pad.numel() // 8, dtype=torch.uint8, device=d.device)
        pv = pad.view(-1, 8)
        for k in range(8):
            byte |= pv[:, k].to(torch.uint8) << k
        gbits_buf[g0 // 8:g0 // 8 + byte.numel()] |= byte
    return g, s_, l_


def _timed(fn, reps):
    """Median-able lists of call and main-kernel times (HIP events)."""
    import torch
    from bit_exact_xor_amd import dcr
    ms, kms = [], []
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[2].record()
        e[3].record()         # creates the events the library records into
        dcr.dcr_set_kernel_events(e[2], e[3])
        e[0].record()
        fn()
        e[1].record()
        torch.cuda.synchronize()
        dcr.dcr_set_kernel_events(None, None)
        ms.append(e[0].elapsed_time(e[1]))
        kms.append(e[2].elapsed_time(e[3]))
    return ms, kms

# ------------------------------------------------------------ HBM traffic
#
# rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE (one counter per run) give
# KiB per dispatch.  Each counter is scaled by what it reads for a plain
# device copy of known size (bench.py --copy-probe).  The scaled bytes per
# launch are kept in a summary under profiles/ (one per workload) together
# with the SHA-256 of the kernel sources they were measured on; the bench
# reports them only while those sources are unchanged, else null.

KERNEL_SRCS = [os.path.join(ROOT, "bit_exact_xor_amd", "csrc", "dcr_kernels.hip"),
               os.path.join(ROOT, "bit_exact_xor_amd", "csrc", "dcr_internal.h")]
TRAFFIC_FILES = {"llama8b_tp4": "encode_apply_llama8b_tp4_hbm_traffic.md",
                 HEADLINE: "encode_apply_qwen3_30b_hot_block_scaled_hbm_traffic.md",
                 "qwen3_30b_ep8_beta": "encode_apply_qwen3_30b_ep8_beta_hbm_traffic.md",
                 "receiver_share_240GB": "apply_receiver_share_240gb_hbm_traffic.md"}
TRAFFIC_TAG = "traffic-json:"
# the main kernel of each op, as rocprofv3 names it (dispatches alternate
# between the two ops of a kernel: DELTA / RETRY encodes, apply / retry)
PMC_KERNELS = {"encode": ("encode_direct_kernel<2,", 0), "encode_retry": ("encode_direct_kernel<2,", 1),
               "apply": ("apply_small_kernel", 0), "retry": ("apply_small_kernel", 1)}


def measured_traffic(key, op):
    """HBM bytes per launch of op's main kernel on workload `key` from the
    committed counter summary, or None when there is none or the kernel
    source has changed since."""
    name = TRAFFIC_FILES.get(key)
    if not name:
        return None
    try:
        with open(os.path.join(ROOT, "profiles", name)) as f:
            line = next(ln for ln in f if ln.strip().startswith(TRAFFIC_TAG))
    except (OSError, StopIteration):
        return None
    rec = json.loads(line.strip()[len(TRAFFIC_TAG):])
    if rec.get("source_sha256") != _src_sha256():
        return None
    return rec["bytes_per_launch"].get(op)


def pmc_report(d, key):
    """Markdown summary of four rocprofv3 --pmc runs under d: pmc_FETCH_SIZE and
    pmc_WRITE_SIZE of `bench.py --only key`, pmc_copy_FETCH_SIZE and
    pmc_copy_WRITE_SIZE of bench.py --copy-probe (3 copies of a known size)."""
    import glob

    def rows(sub):
        (path,) = glob.glob(os.path.join(d, sub, "*_counter_collection.csv"))
        return _pmc_rows(path)

    def per_kernel(rs, name):
        out = {}
        for r in rs:
            if name in r["Kernel_Name"].replace(" ", ""):
                out.setdefault(int(r["Dispatch_Id"]), 0.0)
                out[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
        return [out[k] for k in sorted(out)]

    factors = {}
    copy_bytes = None
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        v = per_kernel(rows(f"pmc_copy_{c}"), "copyBuffer")
        kib = float(np.mean(v))
        with open(os.path.join(d, f"pmc_copy_{c}.log")) as f:
            probe = json.loads(next(ln for ln in f if ln.startswith("{\"copy_probe_bytes\"")))
        copy_bytes = probe["copy_probe_bytes"]
        factors[c] = copy_bytes / (kib * 1024.0)
    ops = PMC_KERNELS if key != "receiver_share_240GB" else {k: v for k, v in PMC_KERNELS.items()
                                                             if k in ("apply", "retry")}
    table, per_launch = [], {}
    for op, (k, parity) in ops.items():
        got = {}
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            v = per_kernel(rows(f"pmc_{c}"), k.replace(" ", ""))
            if key == "receiver_share_240GB":
                # the apply runs, then as many retry runs (an odd --steps)
                v = v[:len(v) // 2] if op == "apply" else v[len(v) // 2:]
            else:
                v = v[parity::2]
            got[c] = (len(v), float(np.mean(v)) if v else float("nan"))
        fb = got["FETCH_SIZE"][1] * 1024 * factors["FETCH_SIZE"]
        wb = got["WRITE_SIZE"][1] * 1024 * factors["WRITE_SIZE"]
        per_launch[op] = int(round(fb + wb))
        table.append(f"| {op} | `{k.rstrip('<,')}` | {got['FETCH_SIZE'][0]} | {got['FETCH_SIZE'][1]:.0f} | "
                     f"{got['WRITE_SIZE'][1]:.0f} | {fb / 1e9:.3f} | {wb / 1e9:.3f} | {(fb + wb) / 1e9:.3f} |")
    out = [f"Copy calibration ({copy_bytes / 2**30:.0f} GiB device copy read and written): "
           f"FETCH_SIZE x {factors['FETCH_SIZE']:.4f}, WRITE_SIZE x {factors['WRITE_SIZE']:.4f}.", "",
           "| op | kernel | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | read GB | written GB | HBM GB / launch |",
           "|---|---|---|---|---|---|---|---|", *table, "",
           TRAFFIC_TAG + " " + json.dumps({"source_sha256": _src_sha256(), "bytes_per_launch": per_launch,
                                            "factors": factors})]
    return "\n".join(out)


def measure_ceiling(buf, dev, reps=3, rmw=None):
    """Best of `reps`: one streaming read of `buf` (the probe kernel of the
    synthetic-input library: 128-bit non-temporal loads, nothing written), a
    4 GiB device-to-device copy (torch; read + write counted) and a 4 GiB
    fill (torch; write only).  With `rmw` = (canonical buffer, group bits,
    touched groups, touched lines): best of four runs of the synthetic
    library's read-modify-write probe over the groups an apply patches (an
    even count, so the buffer ends as it started)."""
    import torch
    from bit_exact_xor_amd import synth
    ev = lambda: torch.cuda.Event(enable_timing=True)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    rd = []
    for _ in range(reps):
        a, b = ev(), ev()
        a.record()
        nread = synth.read_probe_gpu(buf, sink)
        b.record()
        torch.cuda.synchronize()
        rd.append(a.elapsed_time(b))
    n = 1 << 32
    src = buf[:n] if buf.numel() >= 2 * n else buf[: buf.numel() // 2]
    dst = torch.empty_like(src)
    cp = []
    for _ in range(reps):
        a, b = ev(), ev()
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        cp.append(a.elapsed_time(b))
    wr = []
    for _ in range(reps):
        a, b = ev(), ev()
        a.record()
        dst.zero_()
        b.record()
        torch.cuda.synchronize()
        wr.append(a.elapsed_time(b))
    del dst
    torch.cuda.empty_cache()
    read_gbps = nread / (min(rd) * 1e-3) / 1e9
    copy_gbps = 2 * src.numel() / (min(cp) * 1e-3) / 1e9
    write_gbps = src.numel() / (min(wr) * 1e-3) / 1e9
    out = {"read_GBps": round(read_gbps, 1), "write_GBps": round(write_gbps, 1), "copy_GBps": round(copy_gbps, 1),
           "read_frac_of_peak": round(read_gbps / PEAK_HBM_GBPS, 4),
           "how": f"streaming read of {nread / 1e9:.2f} GB (128-bit non-temporal loads), a "
                  f"{src.numel() / 2**30:.0f} GiB torch device copy (read + write counted) and fill, best of {reps}"}
    if rmw is not None:
        cbuf, bits, n_groups, n_lines = rmw
        rm = []
        for _ in range(4):
            a, b = ev(), ev()
            a.record()
            synth.rmw_probe_gpu(cbuf, bits)
            b.record()
            torch.cuda.synchronize()
            rm.append(a.elapsed_time(b))
        ms = min(rm)
        out["rmw"] = {"ms": round(ms, 4), "groups": n_groups, "lines": n_lines,
                      "line_GBps": round(2 * LINE * n_lines / (ms * 1e-3) / 1e9, 1),
                      "how": "read-modify-write (XOR) of the 16-byte groups an apply of this stream patches, "
                             "in place in the canonical buffer, no records read; one thread per 16 consecutive "
                             "groups; best of 4 (even: the buffer ends unchanged); line_GBps counts a 128-byte "
                             "line read and written per touched line"}
        rl = []
        for _ in range(4):
            a, b = ev(), ev()
            a.record()
            synth.rmw_probe_gpu(cbuf, bits, whole_lines=True)
            b.record()
            torch.cuda.synchronize()
            rl.append(a.elapsed_time(b))
        ms = min(rl)
        out["rmw_lines"] = {"ms": round(ms, 4), "lines": n_lines,
                            "line_GBps": round(2 * LINE * n_lines / (ms * 1e-3) / 1e9, 1),
                            "how": "the same groups patched with every touched 128-byte line read and written "
                                   "whole (one thread per 16-byte group; the buffer is 256-byte aligned, so its "
                                   "lines are the GPU's), no records read; best of 4"}
    return out


def _code_text(text):
    """C++ source text without its comments and with its blank space collapsed:
    what the compiler sees of it (the sources hold no comment markers inside
    string literals)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def _src_sha256(paths=None):
    """SHA-256 over the code of the kernel sources the counters depend on (the
    kernels and the constants they are built with): an edit to a comment
    leaves the measured kernels, and so the hash, unchanged."""
    import hashlib
    h = hashlib.sha256()
    for path in (paths or KERNEL_SRCS):
        with open(path) as f:
            h.update(_code_text(f.read()).encode())
    return h.hexdigest()


def _pmc_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def pmc_dump(d):
    """Markdown table: per main kernel and op (dispatches alternate DELTA /
    RETRY, apply / retry), the per-dispatch average of every counter found in
    the runs DIR/pmc_*/bench_counter_collection.csv."""
    import glob
    ops = [("encode", "encode_direct_kernel", 0), ("encode_retry", "encode_direct_kernel", 1),
           ("apply", "apply_small_kernel", 0), ("retry", "apply_small_kernel", 1),
           ("fix-up (DELTA)", "encode_fixup_kernel", 0)]
    vals = {}
    counters = []
    for path in sorted(glob.glob(os.path.join(d, "pmc_*", "bench_counter_collection.csv"))):
        per = {}
        for r in _pmc_rows(path):
            key = (r["Kernel_Name"], int(r["Dispatch_Id"]), r["Counter_Name"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        for (kn, disp, cn), v in per.items():
            if cn not in counters:
                counters.append(cn)
            vals.setdefault((kn, cn), []).append((disp, v))
    lines = ["| counter | " + " | ".join(o for o, _, _ in ops) + " |", "|---|" + "---|" * len(ops)]
    for cn in counters:
        row = []
        for _, k, par in ops:
            xs = sorted(v for (kn, c), v in vals.items() if k in kn and c == cn for v in v)
            xs = [v for _, v in sorted(xs)][par::2]
            row.append(f"{np.mean(xs):.4g}" if xs else "-")
        lines.append(f"| `{cn}` | " + " | ".join(row) + " |")
    return "\n".join(lines)


def fmt_dirents(d):
    d = np.asarray(d, dtype=np.uint8).reshape(-1, 32)
    out = []
    for e in d:
        out.append(dict(t=int(e[0:4].view("<u4")[0]), c=int(e[4:8].view("<u4")[0]),
                        K=int(e[8:12].view("<u4")[0]), kind=int(e[12]), hi_mode=int(e[13]),
                        off=int(e[16:24].view("<u8")[0]), size=int(e[24:28].view("<u4")[0]),
                        H=int(e[28:32].view("<u4")[0])))
    return out


if __name__ == "__main__":
    main()
