#!/usr/bin/env python3
"""Benchmark: bit-exact delta refit hot path on one MI355X.

Workload: a Llama-style 8B BF16 checkpoint (hidden 4096, 32 layers, FFN 14336,
32 q / 8 kv heads x 128, vocab 128256; 8.03 B parameters, 16.06 GB) trained
with tensor parallelism 4 (vocab-parallel embed / lm_head, fused QKV routed to
overwrite records, fused gate/up column split, row-split o / down), 1 % of the
stored values changed uniformly at random (+-1 BF16 ulp).  Inputs are
synthetic and seeded, generated on the GPU; nothing is read from disk.

One step = one pass of the whole hot path:
  encode (DELTA)   bit-diff + projection + routing + compaction + records (staged),
                   then the fix-up pass (prefix scan, staged records moved into place)
  apply            the DELTA stream in place on the receiver's canonical tensors
  encode (RETRY)   the whole change set as overwrites
  retry            the RETRY stream re-applied as overwrites
value = canonical BF16 bytes scanned per step / step time (GB/s).

Prints one JSON line (rank 0).  --gpus above 1 is refused: the path is a
single-GPU one.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
LINE = 128   # bytes an apply reads per touched line (L2 line fill)
SECTOR = 32  # bytes an apply writes back per dirty sector (the L2 writes dirty 32-byte sectors)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle leg")
    ap.add_argument("--cpu-reps", type=int, default=4, help="oracle steps timed on the sample")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the measurements outside the step (partial retry, index lists, receiver layout, "
                         "pipelined transfer); for profiler runs")
    ap.add_argument("--copy-probe", type=float, default=0.0, metavar="GIB",
                    help="only run a plain device copy of this many GiB, 3 times (counter calibration)")
    ap.add_argument("--pmc-report", metavar="DIR",
                    help="summarise rocprofv3 FETCH_SIZE / WRITE_SIZE runs found under DIR and exit")
    ap.add_argument("--lists-cfg5", action="store_true",
                    help="only compare the bitmap and index-list streams on config 5's NVFP4 region (40 GB at "
                         "0.085 %% bytes) and a 29 GB slice of its BF16 region (3 %%); print one JSON line")
    ap.add_argument("--configs", action="store_true",
                    help="only time encode / apply / retry on the other workloads at full size (4096x4096 "
                         "tensor at 1 %%; Qwen3-30B-A3B-shaped EP=8 at 3 %% Beta(2,60) rates; the same at 5 %% "
                         "hot rows, block-scaled; the 240 GB receiver share, apply and retry only); print one "
                         "JSON line")
    ap.add_argument("--configs-only", default=None, metavar="NAME",
                    help="with --configs: only the workload whose name contains NAME (for profiler runs)")
    ap.add_argument("--pmc-dump", metavar="DIR",
                    help="per-kernel averages of every counter in the rocprofv3 runs under DIR/pmc_*; exit")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.pmc_report:
        print(pmc_report(args.pmc_report))
        return
    if args.pmc_dump:
        print(pmc_dump(args.pmc_dump))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py: --gpus {args.gpus}: the library runs the hot path on one GPU only "
              "(no cross-GPU sharding or collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_exact_xor_amd import dcr, synth

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
    if args.configs:
        print(json.dumps(bench_configs(dev, only=args.configs_only)), flush=True)
        return

    # ---------------------------------------------------------------- setup
    t0 = time.time()
    lay = synth.llama_layout()
    plan = dcr.dcr_plan_build(lay.tensors, [lay.shard_bytes(s) for s in range(lay.n_shards)], lay.segments)
    dcr.dcr_plan_upload(plan, dev)
    info = plan.info
    log(f"plan: {info.n_tensors} tensors, {info.n_shards} shards, {info.n_chunks} chunks, "
        f"{info.n_pieces} pieces, {info.canonical_bytes / 1e9:.2f} GB canonical "
        f"({time.time() - t0:.1f}s)")
    old_buf, olds = synth.alloc_shards(lay, dev)
    new_buf, news = synth.alloc_shards(lay, dev)
    synth.fill_shards_gpu(lay, olds, 0)
    synth.fill_shards_gpu(lay, news, 1)
    torch.cuda.synchronize()

    def as_i16(views):
        return [v.view(torch.int16) for v in views]

    # receiver: canonical tensors assembled from the old shards with library ops
    canon_old = lay.assemble(as_i16(olds))
    T = lay.tensors
    sizes = [int(T[t]["numel"]) * int(T[t]["elem_bytes"]) for t in range(len(T))]
    offs = np.concatenate([[0], np.cumsum([(s + 255) // 256 * 256 for s in sizes])]).astype(np.int64)
    canon_buf = torch.empty(int(offs[-1]), dtype=torch.uint8, device=dev)
    canon = [canon_buf[int(offs[t]):int(offs[t]) + sizes[t]] for t in range(len(T))]
    for t in range(len(T)):
        canon[t].view(torch.int16).copy_(canon_old[t].reshape(-1))
    del canon_old
    cb = int(info.canonical_bytes)
    payload_cap = int(cb * 0.2) + (1 << 20)
    # workspace with a staging area holding every chunk's slot: no encode
    # tile waits for its predecessors
    ws = dcr.workspace(plan, dev, stage_bytes=int(info.max_payload_bytes))
    delta = dcr.StreamBuffers(plan, dev, dir_bytes=2 * 32 * int(info.n_chunks),
                              payload_bytes=payload_cap)
    retry = dcr.StreamBuffers(plan, dev, dir_bytes=32 * int(info.n_chunks),
                              payload_bytes=payload_cap)
    torch.cuda.synchronize()
    log(f"inputs ready ({time.time() - t0:.1f}s)")

    # ---------------------------------------------------- first step + checks
    # address tables built once (pinned host memory), as a caller that keeps
    # its buffers would
    olds_t, news_t, canon_t = dcr.PtrTable(olds), dcr.PtrTable(news), dcr.PtrTable(canon)

    def encode(sb, mode):
        dcr.dcr_encode(plan, olds_t, news_t, mode, 41, 42, sb.header, sb.dir, sb.payload, sb.result, ws)

    def encode_ws(sb, mode, w):
        dcr.dcr_encode(plan, olds_t, news_t, mode, 41, 42, sb.header, sb.dir, sb.payload, sb.result, w)

    encode(delta, 0)
    encode(retry, 1)
    torch.cuda.synchronize()
    for name, sb in (("delta", delta), ("retry", retry)):
        r = sb.result_host()
        if int(r["status"]) != 0:
            raise SystemExit(f"{name} stream does not fit: {r}")
    hdr = delta.header_host()
    rhdr = retry.header_host()
    n_rec, p_bytes = delta.n_records(), delta.payload_bytes()
    rn_rec, rp_bytes = retry.n_records(), retry.payload_bytes()
    n_changed = int(delta.result_host()["n_changed"])
    flags = torch.zeros(max(n_rec, 1), dtype=torch.uint8, device=dev)
    ares = torch.zeros(32, dtype=torch.uint8, device=dev)

    def apply():
        flags.zero_()
        dcr.dcr_apply(plan, canon_t, hdr, delta.dir, delta.payload, flags, 0, n_rec, 41, ares, ws)

    def do_retry():
        dcr.dcr_apply_overwrite_retry(plan, canon_t, rhdr, retry.dir, retry.payload, 41, ares, ws)

    # apply on old must give new; the retry keeps new; checked on the whole model
    canon_new = lay.assemble(as_i16(news))
    apply()
    torch.cuda.synchronize()
    ok_apply = all(torch.equal(canon[t].view(torch.int16), canon_new[t].reshape(-1)) for t in range(len(T)))
    do_retry()
    torch.cuda.synchronize()
    ok_retry = all(torch.equal(canon[t].view(torch.int16), canon_new[t].reshape(-1)) for t in range(len(T)))
    # touched 128-byte lines and 32-byte sectors (apply traffic model), from old vs new
    touched = touched_sec = 0
    canon_o = lay.assemble(as_i16(olds))
    # one flag per 16-byte group of canon_buf holding a change (the groups an
    # apply patches), for the read-modify-write ceiling below
    n_groups = (int(offs[-1]) // 16 + 127) // 128 * 128
    gflags = torch.zeros(n_groups, dtype=torch.bool, device=dev)
    for t in range(len(T)):
        d = (canon_o[t].reshape(-1) != canon_new[t].reshape(-1))
        n = d.numel()
        ng = (n + 7) // 8
        gd = torch.zeros(ng * 8, dtype=torch.bool, device=dev)
        gd[:n] = d
        gflags[int(offs[t]) // 16:int(offs[t]) // 16 + ng] = gd.view(-1, 8).any(1)
        del gd
        for gran in (LINE, SECTOR):
            per = gran // 2
            full = n // per * per
            cnt = int(d[:full].view(-1, per).any(1).sum()) + (int(d[full:].any()) if full < n else 0)
            if gran == LINE:
                touched += cnt
            else:
                touched_sec += cnt
    del canon_new, canon_o
    gbits = torch.zeros(n_groups // 8, dtype=torch.uint8, device=dev)
    gv = gflags.view(-1, 8)
    for k in range(8):
        gbits |= gv[:, k].to(torch.uint8) << k
    n_touched_groups = int(gflags.sum())
    del gflags, gv
    torch.cuda.empty_cache()
    log(f"first step: apply==new {ok_apply}, retry==new {ok_retry}; {n_rec} records "
        f"{p_bytes / 1e9:.3f} GB payload; retry {rn_rec} records {rp_bytes / 1e9:.3f} GB; "
        f"{n_changed} changed ({n_changed / (cb / 2) * 100:.3f} %)")

    # -------------------------------------------------------------- timing
    ops = ["encode", "apply", "encode_retry", "retry"]
    fns = [lambda: encode(delta, 0), apply, lambda: encode(retry, 1), do_retry]
    for _ in range(args.warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    def pair():
        return (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    ev = [[pair() for _ in ops] for _ in range(args.steps)]      # around each call
    kev = [[pair() for _ in ops] for _ in range(args.steps)]     # around its main kernel (the library records)
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
    op_ms = {op: float(np.mean([ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)]))
             for i, op in enumerate(ops)}
    kern_ms = {op: float(np.mean([kev[s][i][0].elapsed_time(kev[s][i][1]) for s in range(args.steps)]))
               for i, op in enumerate(ops)}
    kern_med = {op: float(np.median([kev[s][i][0].elapsed_time(kev[s][i][1]) for s in range(args.steps)]))
                for i, op in enumerate(ops)}
    ms_per_step = wall * 1e3 / args.steps
    # the stream after timing is still new (each step ends with the retry)
    ok_after = True
    canon_new = lay.assemble(as_i16(news))
    ok_after = all(torch.equal(canon[t].view(torch.int16), canon_new[t].reshape(-1)) for t in range(len(T)))
    del canon_new

    # extras outside the step (skipped for profiling runs, so that every
    # launch of the step kernels in a trace belongs to the step)
    partial_retry = retry_from_delta = index_lists = sharded_apply = pipelined = staging_modes = None
    if not args.no_extras:
        # partial retry after a kill at 50 % of the DELTA records (outside the
        # step): the receiver is set back to old, applies the first half, and the
        # sender re-encodes only the chunks of the unflagged records
        canon_o = lay.assemble(as_i16(olds))
        for t in range(len(T)):
            canon[t].view(torch.int16).copy_(canon_o[t].reshape(-1))
        del canon_o
        flags.zero_()
        dcr.dcr_apply(plan, canon, hdr, delta.dir, delta.payload, flags, 0, n_rec // 2, 41, ares, ws)
        torch.cuda.synchronize()
        pe, pa = [], []
        for _ in range(3):
            a_, b_ = pair()
            a_.record()
            dcr.dcr_encode_retry_partial(plan, olds, news, hdr, delta.dir, flags, 41, 42, retry.header, retry.dir,
                                         retry.payload, retry.result, ws)
            b_.record()
            torch.cuda.synchronize()
            pe.append(a_.elapsed_time(b_))
        pr = retry.result_host()
        ph = retry.header_host()
        for _ in range(3):
            a_, b_ = pair()
            a_.record()
            dcr.dcr_apply_overwrite_retry(plan, canon, ph, retry.dir, retry.payload, 41, ares, ws)
            b_.record()
            torch.cuda.synchronize()
            pa.append(a_.elapsed_time(b_))
        canon_new = lay.assemble(as_i16(news))
        ok_partial = all(torch.equal(canon[t].view(torch.int16), canon_new[t].reshape(-1)) for t in range(len(T)))
        del canon_new
        partial_retry = {"kill_at_records": n_rec // 2, "status": int(pr["status"]), "records": int(pr["n_records"]),
                         "payload_GB": round(int(pr["payload_bytes"]) / 1e9, 4),
                         "full_retry_payload_GB": round(rp_bytes / 1e9, 4),
                         "encode_ms": round(float(np.median(pe)), 4),
                         "full_retry_encode_ms": round(op_ms["encode_retry"], 4),
                         "apply_ms": round(float(np.median(pa)), 4), "full_retry_apply_ms": round(op_ms["retry"], 4),
                         "healed_eq_new": bool(ok_partial)}
        log(f"partial retry at a 50 % kill: {partial_retry}")

        # the RETRY stream written from the step's DELTA stream and old only
        # (outside the step): timed, then applied to old, which must give new
        te = []
        for _ in range(3):
            a_, b_ = pair()
            a_.record()
            dcr.dcr_encode_retry_from_delta(plan, olds, hdr, delta.dir, delta.payload, 0, retry.header, retry.dir,
                                            retry.payload, retry.result, ws)
            b_.record()
            torch.cuda.synchronize()
            te.append(a_.elapsed_time(b_))
        tr = retry.result_host()
        canon_o = lay.assemble(as_i16(olds))
        for t in range(len(T)):
            canon[t].view(torch.int16).copy_(canon_o[t].reshape(-1))
        del canon_o
        dcr.dcr_apply_overwrite_retry(plan, canon, retry.header_host(), retry.dir, retry.payload, 41, ares, ws)
        torch.cuda.synchronize()
        canon_new = lay.assemble(as_i16(news))
        ok_tx = all(torch.equal(canon[t].view(torch.int16), canon_new[t].reshape(-1)) for t in range(len(T)))
        del canon_new
        retry_from_delta = {"status": int(tr["status"]), "records": int(tr["n_records"]),
                            "payload_GB": round(int(tr["payload_bytes"]) / 1e9, 4),
                            "same_size_as_retry": int(tr["payload_bytes"]) == rp_bytes,
                            "encode_ms": round(float(np.median(te)), 4),
                            "full_retry_encode_ms": round(op_ms["encode_retry"], 4),
                            "applied_eq_new": bool(ok_tx)}
        log(f"RETRY stream from the DELTA stream: {retry_from_delta}")

        # index-list layout (encode option, outside the step): the same DELTA
        # change set with low-density records carrying 16-bit indices instead of
        # the bitmap; encoded into the retry buffers, applied to old, checked
        canon_o = lay.assemble(as_i16(olds))
        le, la = [], []
        for _ in range(3):
            a_, b_ = pair()
            a_.record()
            dcr.dcr_encode(plan, olds, news, dcr.MODE_DELTA | dcr.ENC_INDEX_LISTS, 41, 42, retry.header, retry.dir,
                           retry.payload, retry.result, ws)
            b_.record()
            torch.cuda.synchronize()
            le.append(a_.elapsed_time(b_))
        lr = retry.result_host()
        lh = retry.header_host()
        ln = int(lr["n_records"])
        lflags = torch.zeros(max(ln, 1), dtype=torch.uint8, device=dev)
        for _ in range(3):
            for t in range(len(T)):
                canon[t].view(torch.int16).copy_(canon_o[t].reshape(-1))
            lflags.zero_()
            torch.cuda.synchronize()
            a_, b_ = pair()
            a_.record()
            dcr.dcr_apply(plan, canon, lh, retry.dir, retry.payload, lflags, 0, ln, 41, ares, ws)
            b_.record()
            torch.cuda.synchronize()
            la.append(a_.elapsed_time(b_))
        del canon_o
        canon_new = lay.assemble(as_i16(news))
        ok_lists = all(torch.equal(canon[t].view(torch.int16), canon_new[t].reshape(-1)) for t in range(len(T)))
        del canon_new
        index_lists = {"status": int(lr["status"]), "records": ln,
                       "payload_GB": round(int(lr["payload_bytes"]) / 1e9, 4),
                       "bitmap_payload_GB": round(p_bytes / 1e9, 4), "encode_ms": round(float(np.median(le)), 4),
                       "bitmap_encode_ms": round(op_ms["encode"], 4), "apply_ms": round(float(np.median(la)), 4),
                       "bitmap_apply_ms": round(op_ms["apply"], 4), "apply_eq_new": bool(ok_lists)}
        log(f"index-list layout: {index_lists}")

        # apply straight into a receiver that stores the model as TP=2 engine
        # shards (outside the step): the DELTA stream through the receiver plan
        lay_r = synth.llama_layout(tp=2)
        rplan = dcr.dcr_plan_build(lay_r.tensors, [lay_r.shard_bytes(s) for s in range(lay_r.n_shards)],
                                   lay_r.segments)
        dcr.dcr_plan_upload(rplan, dev)
        rws = dcr.workspace(rplan, dev)
        canon_o = lay.assemble(as_i16(olds))
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
        got = lay_r.assemble([x.view(torch.int16) for x in rsh])
        canon_new = lay.assemble(as_i16(news))
        ok_sharded = all(torch.equal(got[t].reshape(-1), canon_new[t].reshape(-1)) for t in range(len(T)))
        del got, canon_new, rbuf, rsh, rws
        torch.cuda.empty_cache()
        sharded_apply = {"receiver": "the same model as TP=2 engine shards (325 shards, 744 833 pieces)",
                         "apply_ms": round(float(np.median(sa)), 4), "canonical_apply_ms": round(op_ms["apply"], 4),
                         "eq_new": bool(ok_sharded)}
        log(f"apply into a TP=2 receiver layout: {sharded_apply}")

        pipelined = pipelined_transfer(plan, lay, olds, news, canon, as_i16, ws, delta, n_rec, p_bytes, dev,
                                       op_ms["encode"], op_ms["apply"])
        log(f"pipelined transfer through pinned host memory: {pipelined}")

        # staging area sizes: the whole worst case (the step's launch
        # configuration), windows of fix-up blocks in 4 GiB and 1 GiB, and
        # none (in-order look-back); each stream compared with the step's
        staging_modes = {"window_stage_bytes": int(info.window_stage_bytes),
                         "full_stage_bytes": int(info.max_payload_bytes)}
        ref = (delta.header.clone(), delta.dir[:32 * n_rec].clone(), delta.payload[:p_bytes].clone())
        del ws
        torch.cuda.empty_cache()
        for name, sbytes in (("full", int(info.max_payload_bytes)), ("window_4GiB", 4 << 30),
                             ("window_1GiB", 1 << 30), ("in_order", 0)):
            wsm = dcr.workspace(plan, dev, stage_bytes=sbytes)
            tm = []
            for _ in range(4):
                a_, b_ = pair()
                a_.record()
                encode_ws(delta, 0, wsm)
                b_.record()
                torch.cuda.synchronize()
                tm.append(a_.elapsed_time(b_))
            same = (torch.equal(delta.header, ref[0]) and torch.equal(delta.dir[:32 * n_rec], ref[1])
                    and torch.equal(delta.payload[:p_bytes], ref[2]))
            staging_modes[name] = {"stage_GB": round(sbytes / 1e9, 3), "encode_ms": round(float(np.median(tm[1:])), 3),
                                   "stream_eq": bool(same)}
            del wsm
            torch.cuda.empty_cache()
        ws = dcr.workspace(plan, dev, stage_bytes=int(info.max_payload_bytes))
        del ref
        log(f"staging area sizes: {staging_modes}")

    enc_bytes = 2 * cb + 32 * n_rec + p_bytes
    renc_bytes = 2 * cb + 32 * rn_rec + rp_bytes
    app_bytes = 32 * n_rec + p_bytes + LINE * touched + SECTOR * touched_sec
    ret_bytes = 32 * rn_rec + rp_bytes + LINE * touched + SECTOR * touched_sec
    alg = {"encode": enc_bytes, "apply": app_bytes, "encode_retry": renc_bytes, "retry": ret_bytes}
    # what the op's main kernel itself moves: the encode tile kernel reads the
    # shards and writes the records (the fix-up pass writes the directory)
    kalg = {"encode": 2 * cb + p_bytes, "apply": app_bytes, "encode_retry": 2 * cb + rp_bytes,
            "retry": ret_bytes}
    per_op = {}
    kname = {"encode": "encode_direct_kernel", "encode_retry": "encode_direct_kernel", "apply": "apply_small_kernel",
             "retry": "apply_small_kernel"}
    for op in ops:
        gbps = alg[op] / (op_ms[op] * 1e-3) / 1e9
        kgbps = kalg[op] / (kern_ms[op] * 1e-3) / 1e9
        per_op[op] = {"ms": round(op_ms[op], 4), "alg_GB": round(alg[op] / 1e9, 4),
                      "alg_GBps": round(gbps, 1), "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
                      "scanned_GBps": round(cb / (op_ms[op] * 1e-3) / 1e9, 1),
                      "kernel": kname[op], "kernel_ms": round(kern_ms[op], 4),
                      "kernel_ms_median": round(kern_med[op], 4),
                      "kernel_alg_GB": round(kalg[op] / 1e9, 4), "kernel_alg_GBps": round(kgbps, 1)}
    # the dominant kernel: its algorithmic bytes over its own launch duration
    dom = max(ops, key=lambda o: kern_ms[o])
    roof = {"bound": "hbm", "kernel": kname[dom], "op": dom, "achieved": per_op[dom]["kernel_alg_GBps"],
            "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(per_op[dom]["kernel_alg_GBps"] / PEAK_HBM_GBPS, 4),
            "traffic": measured_traffic(dom)}

    # measured ceilings on this GPU: a streaming read and a device copy
    ceiling = measure_ceiling(old_buf, dev, rmw=(canon_buf, gbits, n_touched_groups, touched))
    for op in ops:
        per_op[op]["kernel_frac_of_read_ceiling"] = round(per_op[op]["kernel_alg_GBps"] / ceiling["read_GBps"], 4)
    # apply / retry against the bare patch of the same groups (no records read)
    for op in ("apply", "retry"):
        per_op[op]["kernel_frac_of_rmw_ceiling"] = round(ceiling["rmw"]["ms"] / kern_ms[op], 4)

    # ------------------------------------------------------- CPU baseline
    cpu = None
    parity_sample = None
    if not args.no_cpu_baseline:
        cpu, parity_sample = cpu_baseline(lay, delta, hdr, args.cpu_reps)

    value = cb / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": "encode & apply GB/s of BF16 weights scanned; % of MI355X HBM peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u16",
        "data": "synthetic, seeded (GPU-generated shards)",
        "config": {"workload": "llama-8B-shaped BF16 checkpoint, TP=4 trainer shards, fused QKV -> overwrite, "
                               "1% uniform +-1ulp changes",
                   "canonical_GB": round(cb / 1e9, 3), "tensors": int(info.n_tensors),
                   "shards": int(info.n_shards), "chunks": int(info.n_chunks), "pieces": int(info.n_pieces),
                   "changed_frac": round(n_changed / (cb / 2), 6),
                   "step": "encode(DELTA)+apply+encode(RETRY)+retry"},
        "ops": per_op,
        "streams": {"delta_records": n_rec, "delta_payload_GB": round(p_bytes / 1e9, 4),
                    "retry_records": rn_rec, "retry_payload_GB": round(rp_bytes / 1e9, 4),
                    "touched_128B_lines": touched, "touched_32B_sectors": touched_sec},
        "checks": {"apply_eq_new": bool(ok_apply), "retry_eq_new": bool(ok_retry),
                   "after_timing_eq_new": bool(ok_after), "oracle_sample": parity_sample},
        "partial_retry": partial_retry,
        "retry_from_delta": retry_from_delta,
        "index_lists": index_lists,
        "sharded_apply": sharded_apply,
        "pipelined": pipelined,
        "staging_modes": staging_modes,
        "roofline": roof,
        "ceiling": ceiling,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


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


def lists_cfg5(dev, reps=3):
    """Bitmap against index-list streams on config 5's two regions (identity
    layouts: shard i = tensor i, so the old shards are the canonical old
    tensors): stream bytes, encode and apply times (median of reps), and the
    weights after an odd number of XOR applies checked against new."""
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


def _op_stats(ms, kms, alg, scanned):
    return {"ms": round(float(np.median(ms)), 4), "kernel_ms": round(float(np.median(kms)), 4),
            "alg_GB": round(alg / 1e9, 4), "kernel_alg_GBps": round(alg / (np.median(kms) * 1e-3) / 1e9, 1),
            "hbm_frac": round(alg / (np.median(kms) * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "scanned_GBps": round(scanned / (np.median(ms) * 1e-3) / 1e9, 1)}


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


def _bench_layout(lay, dev, reps, host_values=None):
    """Encode DELTA / RETRY (staged when the staging area fits), apply and
    retry of one full-size layout whose canonical tensors are contiguous
    shard runs: the receiver is a copy of the old shard buffer, patched in
    place through per-tensor views."""
    import torch
    from bit_exact_xor_amd import dcr, synth
    T = lay.tensors
    plan = dcr.dcr_plan_build(T, [lay.shard_bytes(s) for s in range(lay.n_shards)], lay.segments)
    dcr.dcr_plan_upload(plan, dev)
    info = plan.info
    cb = int(info.canonical_bytes)
    old_buf, olds = synth.alloc_shards(lay, dev)
    new_buf, news = synth.alloc_shards(lay, dev)
    if host_values is not None:
        for dst, src in zip(olds, host_values[0]):
            dst.copy_(torch.from_numpy(src.view(np.uint8)))
        for dst, src in zip(news, host_values[1]):
            dst.copy_(torch.from_numpy(src.view(np.uint8)))
    else:
        synth.fill_shards_gpu(lay, olds, 0)
        synth.fill_shards_gpu(lay, news, 1)
    torch.cuda.synchronize()
    cap = int(cb * 0.16) + (1 << 24)
    delta = dcr.StreamBuffers(plan, dev, dir_bytes=2 * 32 * int(info.n_chunks), payload_bytes=cap)
    retry = dcr.StreamBuffers(plan, dev, dir_bytes=2 * 32 * int(info.n_chunks), payload_bytes=cap)
    free, _ = torch.cuda.mem_get_info()
    stage = int(info.max_payload_bytes)
    # the receiver copy and the group bits come after the encodes
    staged = stage + cb + (8 << 30) < int(free)
    ws = dcr.workspace(plan, dev, stage if staged else 0)

    olds_t, news_t = dcr.PtrTable(olds), dcr.PtrTable(news)

    def enc(sb, mode):
        dcr.dcr_encode(plan, olds_t, news_t, mode, 41, 42, sb.header, sb.dir, sb.payload, sb.result, ws)

    enc(delta, 0)
    enc(retry, 1)
    torch.cuda.synchronize()
    for nm, sb in (("delta", delta), ("retry", retry)):
        r = sb.result_host()
        if int(r["status"]) != 0:
            raise SystemExit(f"{lay.name} {nm} stream does not fit: {r}")
    n_rec, p_bytes = delta.n_records(), delta.payload_bytes()
    rn_rec, rp_bytes = retry.n_records(), retry.payload_bytes()
    n_changed = int(delta.result_host()["n_changed"])
    e_ms, e_kms = _timed(lambda: enc(delta, 0), reps)
    r_ms, r_kms = _timed(lambda: enc(retry, 1), reps)
    del ws
    torch.cuda.empty_cache()
    ws = dcr.workspace(plan, dev)
    hdr, rhdr = delta.header_host(), retry.header_host()
    recv = old_buf.clone()
    canon = _views(lay, recv, [recv[s.data_ptr() - old_buf.data_ptr():][:s.numel()] for s in olds])
    ov = _views(lay, old_buf, olds)
    nv = _views(lay, new_buf, news)
    gbits = torch.zeros((old_buf.numel() // 16 + 127) // 128 * 16, dtype=torch.uint8, device=dev)
    n_groups, n_sec, n_lines = _touched(ov, nv, gbits, [v.data_ptr() - old_buf.data_ptr() for v in ov])
    flags = torch.zeros(max(n_rec, 1), dtype=torch.uint8, device=dev)
    res = torch.zeros(32, dtype=torch.uint8, device=dev)

    canon_t = dcr.PtrTable(canon)

    def apply():
        flags.zero_()
        dcr.dcr_apply(plan, canon_t, hdr, delta.dir, delta.payload, flags, 0, n_rec, 41, res, ws)

    def do_retry():
        dcr.dcr_apply_overwrite_retry(plan, canon_t, rhdr, retry.dir, retry.payload, 41, res, ws)

    apply()
    torch.cuda.synchronize()
    ok_apply = all(torch.equal(a, b) for a, b in zip(canon, nv))
    a_ms, a_kms = [], []
    t_ms, t_kms = [], []
    for _ in range(reps):
        x = _timed(apply, 1)
        y = _timed(do_retry, 1)     # back to new: every apply starts from the same state
        a_ms += x[0]
        a_kms += x[1]
        t_ms += y[0]
        t_kms += y[1]
    ok_retry = all(torch.equal(a, b) for a, b in zip(canon, nv))
    # read-modify-write ceiling over the touched groups (even count: restored)
    rm = []
    for _ in range(4):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        synth.rmw_probe_gpu(recv, gbits)
        e1.record()
        torch.cuda.synchronize()
        rm.append(e0.elapsed_time(e1))
    rmw_ms = min(rm)
    graph = None
    if cb < (1 << 30):
        # small workloads are launch-bound: encode (staged) + apply captured
        # once in a HIP graph and replayed, against the same calls eager
        gsb = dcr.StreamBuffers(plan, dev, dir_bytes=2 * 32 * int(info.n_chunks), payload_bytes=cap)
        wsg = dcr.workspace(plan, dev, stage if staged else 0)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            dcr.dcr_encode(plan, olds_t, news_t, 0, 41, 42, gsb.header, gsb.dir, gsb.payload, gsb.result, wsg)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            dcr.dcr_encode(plan, olds_t, news_t, 0, 41, 42, gsb.header, gsb.dir, gsb.payload, gsb.result, wsg)
            flags.zero_()
            dcr.dcr_apply(plan, canon_t, hdr, gsb.dir, gsb.payload, flags, 0, n_rec, 41, res, ws)
        gsb.dir.fill_(0xEE)
        g.replay()
        torch.cuda.synchronize()
        same = (torch.equal(gsb.header, delta.header) and torch.equal(gsb.dir[:32 * n_rec], delta.dir[:32 * n_rec])
                and torch.equal(gsb.payload[:p_bytes], delta.payload[:p_bytes]))
        gt, et = [], []
        for _ in range(20):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            gt.append(e0.elapsed_time(e1))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            enc(delta, 0)
            apply()
            e1.record()
            torch.cuda.synchronize()
            et.append(e0.elapsed_time(e1))
        graph = {"encode_apply_replay_ms": round(float(np.median(gt)), 4),
                 "encode_apply_eager_ms": round(float(np.median(et)), 4), "stream_eq_eager": bool(same)}
        del g, gsb, wsg
    # the RETRY stream written from the DELTA stream, into the retry buffers
    # (after the retry timings): the same stream again, checked by its sizes,
    # header and the sums of its 64-bit words
    def words(t, n):
        return int(t[:n].view(torch.int64).sum()) if n else 0
    want = (words(retry.dir, 32 * rn_rec), words(retry.payload, rp_bytes))
    x_ms, _ = _timed(lambda: dcr.dcr_encode_retry_from_delta(plan, olds_t, hdr, delta.dir, delta.payload, 0,
                                                             retry.header, retry.dir, retry.payload, retry.result,
                                                             ws), reps)
    xr = retry.result_host()
    x_same = (int(xr["status"]) == 0 and retry.n_records() == rn_rec and retry.payload_bytes() == rp_bytes
              and np.array_equal(retry.header_host(), rhdr)
              and (words(retry.dir, 32 * rn_rec), words(retry.payload, rp_bytes)) == want)
    app_alg = 32 * n_rec + p_bytes + LINE * n_lines + SECTOR * n_sec
    ret_alg = 32 * rn_rec + rp_bytes + LINE * n_lines + SECTOR * n_sec
    out = {"canonical_GB": round(cb / 1e9, 3), "tensors": int(info.n_tensors), "chunks": int(info.n_chunks),
           "changed_frac_of_elements": round(n_changed / sum(int(t["numel"]) for t in T), 6),
           "staged_encode": bool(staged),
           "delta": {"records": n_rec, "payload_GB": round(p_bytes / 1e9, 4)},
           "retry_stream": {"records": rn_rec, "payload_GB": round(rp_bytes / 1e9, 4)},
           "touched": {"groups16": n_groups, "sectors32": n_sec, "lines128": n_lines},
           "encode": _op_stats(e_ms, e_kms, 2 * cb + p_bytes, cb),
           "encode_retry": _op_stats(r_ms, r_kms, 2 * cb + rp_bytes, cb),
           "apply": _op_stats(a_ms, a_kms, app_alg, cb),
           "retry": _op_stats(t_ms, t_kms, ret_alg, cb),
           "rmw_ceiling_ms": round(rmw_ms, 4),
           "retry_from_delta": {"ms": round(float(np.median(x_ms)), 4), "same_stream": bool(x_same)},
           "checks": {"apply_eq_new": bool(ok_apply), "retry_eq_new": bool(ok_retry)}}
    if graph is not None:
        out["graph"] = graph
    for op in ("apply", "retry"):
        out[op]["kernel_frac_of_rmw_ceiling"] = round(rmw_ms / out[op]["kernel_ms"], 4)
    del recv, canon, canon_t, olds_t, news_t, old_buf, new_buf, olds, news, delta, retry, ws, gbits, flags
    torch.cuda.empty_cache()
    return out


def _bench_cfg5(dev, reps, window=256):
    """The 240 GB receiver share: streams built window by window (the new
    values never fit beside the receiver), then the DELTA apply of every
    record and the overwrite retry of every record, timed in place."""
    import torch
    from bit_exact_xor_amd import dcr, synth
    lay = synth.config5_layout()
    T = lay.tensors
    plan_full = dcr.dcr_plan_build(T, [lay.shard_bytes(s) for s in range(lay.n_shards)], lay.segments)
    dcr.dcr_plan_upload(plan_full, dev)
    n_chunks = int(plan_full.info.n_chunks)
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
                # this window's old / new bytes, flagged at the receiver's offsets
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
    flags = torch.zeros(n_rec, dtype=torch.uint8, device=dev)

    canon_t = dcr.PtrTable(canon)

    def apply():
        flags.zero_()
        dcr.dcr_apply(plan_full, canon_t, hdr, dir_buf, payload, flags, 0, n_rec, 5, res, ws)

    # every rep applies the same XOR stream: old -> new -> old ...
    a_ms, a_kms = _timed(apply, 2 * ((reps + 1) // 2) + 1)
    ok_apply = eq_new()
    rm = []
    for _ in range(4):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        synth.rmw_probe_gpu(cbuf, gbits)
        e1.record()
        torch.cuda.synchronize()
        rm.append(e0.elapsed_time(e1))
    del dir_buf, payload, flags
    torch.cuda.empty_cache()
    rdir = torch.empty(32 * n_chunks, dtype=torch.uint8, device=dev)
    rpay = torch.empty(28 * 10**9, dtype=torch.uint8, device=dev)
    rhdr, rn, rpb, _ = build(1, rdir, rpay, False)
    t_ms, t_kms = _timed(lambda: dcr.dcr_apply_overwrite_retry(plan_full, canon_t, rhdr, rdir, rpay, 5, res, ws),
                         reps)
    ok_retry = eq_new()
    rmw_ms = min(rm)
    g, s_, l_ = touched
    out = {"canonical_GB": round(cb / 1e9, 3), "tensors": int(plan_full.info.n_tensors), "chunks": n_chunks,
           "delta": {"records": n_rec, "payload_GB": round(p_bytes / 1e9, 4), "changed": changed},
           "retry_stream": {"records": rn, "payload_GB": round(rpb / 1e9, 4)},
           "touched": {"groups16": g, "sectors32": s_, "lines128": l_},
           "apply": _op_stats(a_ms, a_kms, 32 * n_rec + p_bytes + LINE * l_ + SECTOR * s_, cb),
           "retry": _op_stats(t_ms, t_kms, 32 * rn + rpb + LINE * l_ + SECTOR * s_, cb),
           "rmw_ceiling_ms": round(rmw_ms, 4),
           "checks": {"apply_eq_new": bool(ok_apply), "retry_eq_new": bool(ok_retry)},
           "note": "apply-only workload: the streams are built window by window outside the timing"}
    for op in ("apply", "retry"):
        out[op]["kernel_frac_of_rmw_ceiling"] = round(rmw_ms / out[op]["kernel_ms"], 4)
    del cbuf, canon, canon_t, rdir, rpay, t_old, t_new, gbits, ws
    torch.cuda.empty_cache()
    return out


def bench_configs(dev, reps=5, only=None):
    """Encode / apply / retry timings on the other full-size workloads (those
    whose name contains `only`, if given)."""
    import gc
    import torch
    from bit_exact_xor_amd import synth
    out = {"what": "encode/apply/retry kernel and call times (medians, HIP events) on full-size workloads; "
                   "hbm_frac = algorithmic bytes / kernel time / 8 TB/s"}
    lay1 = synth.config1_layout()
    o1, n1, _lr, _pos = synth.config1_values(lay1, lr=synth.CFG1_LR)
    for name, lay, hv in (("tensor_4096x4096_1pct", lay1, ([o1], [n1])),
                          ("qwen3_30b_a3b_ep8_3pct_beta", None, None),
                          ("qwen3_30b_a3b_5pct_hot_block_scaled", None, None)):
        if only and only not in name:
            continue
        if lay is None:
            lay = synth.config3_layout() if "beta" in name else synth.config4_layout()
        log(f"configs: {name}")
        out[name] = _bench_layout(lay, dev, reps, hv)
        gc.collect()
        torch.cuda.empty_cache()
    if only and only not in "receiver_share_240GB":
        return out
    log("configs: receiver_share_240GB")
    free, _ = torch.cuda.mem_get_info()
    need = 240 * 10**9 + 16 * 10**9 + 2 * 10**9 + 26 * 10**9
    if free < need:
        out["receiver_share_240GB"] = {"skipped": f"needs {need / 1e9:.0f} GB of free HBM, "
                                                  f"{free / 1e9:.0f} GB available"}
    else:
        out["receiver_share_240GB"] = _bench_cfg5(dev, reps=3)
    return out


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
    return out


def cpu_baseline(lay, delta, hdr_dev, reps):
    """Time the oracle (single thread) on a bounded sample of the same
    workload: layer 0's attention tensors (q, k, v, o) and input norm.  Also
    compares the oracle's records for that sample with the GPU stream."""
    import torch
    from oracle import oracle as O

    orc = O.get()
    names = lay.tensor_names
    sel = [i for i, n in enumerate(names)
           if n.startswith("model.layers.0.") and ("self_attn" in n or "input_layernorm" in n)]
    segs = lay.segments[np.isin(lay.segments["tensor_id"], sel)].copy()
    shards = sorted(set(int(s) for s in segs["shard_id"]))
    tmap = {t: i for i, t in enumerate(sel)}
    smap = {s: i for i, s in enumerate(shards)}
    segs["tensor_id"] = [tmap[int(t)] for t in segs["tensor_id"]]
    segs["shard_id"] = [smap[int(s)] for s in segs["shard_id"]]
    T = lay.tensors[sel].copy()
    olds = [lay.shard_host(s, 0) for s in shards]
    news = [lay.shard_host(s, 1) for s in shards]
    sample_bytes = int(sum(int(t["numel"]) * int(t["elem_bytes"]) for t in T))
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        rc, h, d, p = orc.encode(T, segs, olds, news, mode=0, base_version=41, new_version=42)
        rc2, rh, rd, rp = orc.encode(T, segs, olds, news, mode=1, base_version=41, new_version=42)
        t1 = time.perf_counter()
        canon = [orc.gather(T, segs, olds, t) for t in range(len(T))]
        t2 = time.perf_counter()
        f = np.zeros(len(d) // 32, np.uint8)
        orc.apply(T, canon, h, d, p, f, expected_base_version=41)
        orc.retry(T, canon, rh, rd, rp, expected_base_version=41)
        t3 = time.perf_counter()
        assert rc == 0 and rc2 == 0
        times.append((t1 - t0) + (t3 - t2))   # the gather of the receiver state is setup
    step_s = float(np.median(times))
    # parity of the sample: the GPU records of these tensors, in order, byte for byte
    gd = delta.dir[: delta.n_records() * 32].cpu().numpy()
    gp = delta.payload[: delta.payload_bytes()].cpu().numpy()
    ents = [e for e in fmt_dirents(gd) if e["t"] in tmap]
    oents = fmt_dirents(d)
    same = len(ents) == len(oents)
    if same:
        for e, o in zip(ents, oents):
            if (tmap[e["t"]], e["c"], e["K"], e["kind"], e["hi_mode"], e["size"], e["H"]) != \
                    (o["t"], o["c"], o["K"], o["kind"], o["hi_mode"], o["size"], o["H"]):
                same = False
                break
            if not np.array_equal(gp[e["off"]:e["off"] + e["size"]], p[o["off"]:o["off"] + o["size"]]):
                same = False
                break
    cpu = {"value": round(sample_bytes / step_s / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"layer-0 attention q/k/v/o + input norm ({sample_bytes / 1e6:.1f} MB BF16, "
                     f"{len(T)} tensors) of the same workload; one step = encode + retry-encode + apply + retry; "
                     f"median of {reps}",
           "step_s": round(step_s, 3)}
    return cpu, {"tensors": len(T), "records": len(oents), "identical": bool(same)}


# ------------------------------------------------------------ HBM traffic
#
# rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE (one counter per run) give
# KiB per dispatch.  Each counter is scaled by what it reads for a plain
# device copy of known size (bench.py --copy-probe).  The scaled bytes per
# launch are kept in a summary under profiles/ together with the SHA-256 of the
# kernel source they were measured on; the bench reports them only while the
# source is unchanged, else null.

KERNEL_SRCS = [os.path.join(ROOT, "bit_exact_xor_amd", "csrc", "dcr_kernels.hip"),
               os.path.join(ROOT, "bit_exact_xor_amd", "csrc", "dcr_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "encode_apply_llama8b_tp4_hbm_traffic.md")
TRAFFIC_TAG = "traffic-json:"


def _src_sha256():
    """SHA-256 over the kernel sources the counters depend on (the kernels and
    the constants they are built with)."""
    import hashlib
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(op):
    """HBM bytes per launch of op's kernel from the committed counter summary,
    or None when that summary is missing or the kernel source has changed."""
    try:
        with open(TRAFFIC_FILE) as f:
            line = next(ln for ln in f if ln.strip().startswith(TRAFFIC_TAG))
    except (OSError, StopIteration):
        return None
    rec = json.loads(line.strip()[len(TRAFFIC_TAG):])
    if rec.get("source_sha256") != _src_sha256():
        return None
    return rec["bytes_per_launch"].get(op)


def _pmc_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def pmc_report(d):
    """Markdown summary of four rocprofv3 --pmc runs under d: pmc_FETCH_SIZE and
    pmc_WRITE_SIZE of bench.py, pmc_copy_FETCH_SIZE and pmc_copy_WRITE_SIZE of
    bench.py --copy-probe (3 copies of a known size)."""
    import glob

    def rows(sub):
        (path,) = glob.glob(os.path.join(d, sub, "*_counter_collection.csv"))
        return _pmc_rows(path)

    def per_kernel(rs, key):
        out = {}
        for r in rs:
            if key in r["Kernel_Name"]:
                out.setdefault(int(r["Dispatch_Id"]), 0.0)
                out[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
        return [out[k] for k in sorted(out)]

    factors = {}
    copy_bytes = None
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        v = per_kernel(rows(f"pmc_copy_{c}"), "copyBuffer")
        kib = float(np.mean(v))
        log_path = os.path.join(d, f"pmc_copy_{c}.log")
        with open(log_path) as f:
            probe = json.loads(next(ln for ln in f if ln.startswith("{\"copy_probe_bytes\"")))
        copy_bytes = probe["copy_probe_bytes"]
        factors[c] = copy_bytes / (kib * 1024.0)
    # dispatch order per step in bench.py: encode DELTA, encode RETRY (first step),
    # then encode DELTA, apply, encode RETRY, retry; kernels alternate
    ops = {"encode": ("encode_direct_kernel", 0), "encode_retry": ("encode_direct_kernel", 1),
           "apply": ("apply_small_kernel", 0), "retry": ("apply_small_kernel", 1)}
    table, per_launch = [], {}
    for op, (k, parity) in ops.items():
        got = {}
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            v = per_kernel(rows(f"pmc_{c}"), k)[parity::2]
            got[c] = (len(v), float(np.mean(v)))
        fb = got["FETCH_SIZE"][1] * 1024 * factors["FETCH_SIZE"]
        wb = got["WRITE_SIZE"][1] * 1024 * factors["WRITE_SIZE"]
        per_launch[op] = int(round(fb + wb))
        table.append(f"| {op} | `{k.rstrip('(')}` | {got['FETCH_SIZE'][0]} | {got['FETCH_SIZE'][1]:.0f} | "
                     f"{got['WRITE_SIZE'][1]:.0f} | {fb / 1e9:.3f} | {wb / 1e9:.3f} | {(fb + wb) / 1e9:.3f} |")
    out = [f"Copy calibration ({copy_bytes / 2**30:.0f} GiB device copy read and written): "
           f"FETCH_SIZE x {factors['FETCH_SIZE']:.4f}, WRITE_SIZE x {factors['WRITE_SIZE']:.4f}.", "",
           "| op | kernel | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | read GB | written GB | HBM GB / launch |",
           "|---|---|---|---|---|---|---|---|", *table, "",
           TRAFFIC_TAG + " " + json.dumps({"source_sha256": _src_sha256(), "bytes_per_launch": per_launch,
                                            "factors": factors})]
    return "\n".join(out)


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
