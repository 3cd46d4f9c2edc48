"""Whole-stream parity of a GPU stream against the oracle -- TEST
INFRASTRUCTURE ONLY (tests, the smoke check and the benchmark's CPU-baseline
leg use it; the product path never does).

Every record of a GPU stream is compared byte for byte with what the oracle
writes for the same inputs.  The oracle is run unchanged, single-threaded per
call, once per group of tensors: a block-scaled tensor together with its
scale tensor, every other tensor alone.  Groups run on a pool of threads: the
oracle is a C library and ctypes releases the interpreter lock for each
call, so the calls run in parallel on the host's cores.

The oracle's inputs are the device shards the GPU encoded, copied to host
memory and cut to the ranges each tensor's segments read (the seeded
generator makes the same bytes on the CPU, but far more slowly).  Within a
group the oracle's records come in (tensor, chunk, kind) order, as in the
GPU stream; every directory entry must match field for field (tensor ids
mapped back, payload offsets taken from the GPU stream, whose offsets are
checked separately to be contiguous) and every record's payload bytes must
match.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import threading
import time

import numpy as np

DIRENT = np.dtype([("t", "<u4"), ("c", "<u4"), ("K", "<u4"), ("kind", "u1"), ("hi_mode", "u1"),
                   ("w", "u1"), ("layout", "u1"), ("off", "<u8"), ("size", "<u4"), ("H", "<u4")])
assert DIRENT.itemsize == 32


def host_cores(cap: int = 16) -> int:
    """Cores this process may run on, at most `cap` (the CPU share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def host_info() -> dict:
    """CPU model, logical CPUs visible, RAM and the oracle's compiler."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    ram = 0
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal:"):
                    ram = int(line.split()[1]) * 1024
                    break
    except OSError:
        pass
    try:
        cc = subprocess.run(["gcc", "--version"], capture_output=True, text=True, timeout=20).stdout.splitlines()[0]
    except Exception:  # noqa: BLE001 - informational only
        cc = "unknown"
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "affinity_cpus": host_cores(1 << 20),
            "ram_GB": round(ram / 1e9, 1), "compiler": cc + " -std=c99 -O2"}


def scale_groups(T, ids=None) -> list:
    """Tensor ids grouped with their scale tensors (ascending within a group,
    groups in ascending order of their first id)."""
    ids = range(len(T)) if ids is None else ids
    idset = set(int(i) for i in ids)
    parent = {i: i for i in idset}

    def find(i):
        while parent[i] != i:
            parent[i] = parent[parent[i]]
            i = parent[i]
        return i

    for i in idset:
        st = int(T[i]["scale_tensor"])
        if st >= 0:
            assert st in idset, "a block-scaled tensor's scale tensor must be checked with it"
            parent[find(i)] = find(st)
    groups = {}
    for i in sorted(idset):
        groups.setdefault(find(i), []).append(i)
    return sorted(groups.values(), key=lambda g: g[0])


def mini_inputs(lay, ids, olds, news, seg_index=None):
    """The inputs of tensors `ids` as a layout of their own: each segment reads
    a private host copy of just the shard range it touches, taken from the
    device shards `olds` / `news` (byte views, one per shard).  Returns
    (tensors, segments, old mini-shards, new mini-shards), tensor ids
    renumbered in the order given."""
    ids = list(ids)
    remap = {t: i for i, t in enumerate(ids)}
    T = lay.tensors[ids].copy()
    for i, t in enumerate(ids):
        st = int(lay.tensors[t]["scale_tensor"])
        if st >= 0:
            T[i]["scale_tensor"] = remap[st]
    rows = []
    for t in ids:
        rows += (seg_index[t] if seg_index is not None else
                 [k for k in range(len(lay.segments)) if int(lay.segments[k]["tensor_id"]) == t])
    segs = []
    so, sn = [], []
    for k in rows:
        g = lay.segments[k]
        nd = int(g["ndim"])
        ext = [int(x) for x in g["extent"][:nd]]
        ss = [int(x) for x in g["shard_stride"][:nd]]
        lo = int(g["shard_off"]) + sum(min(0, (e - 1) * s) for e, s in zip(ext, ss))
        hi = int(g["shard_off"]) + sum(max(0, (e - 1) * s) for e, s in zip(ext, ss)) + 1
        s = int(g["shard_id"])
        w = lay.shard_w[s]
        so.append(olds[s][lo * w:hi * w].cpu().numpy())
        sn.append(news[s][lo * w:hi * w].cpu().numpy())
        g2 = g.copy()
        g2["tensor_id"] = remap[int(g["tensor_id"])]
        g2["shard_id"] = len(segs)
        g2["shard_off"] = int(g["shard_off"]) - lo
        segs.append(g2)
    S = np.array(segs, dtype=lay.segments.dtype) if segs else np.zeros(0, dtype=lay.segments.dtype)
    return T, S, so, sn


class HostStream:
    """A stream in host memory: header, directory entries, payload bytes, and
    the directory rows of each tensor (records are ordered by tensor)."""

    def __init__(self, hdr, d, p, p_len=None):
        """p may be None when only the directory is checked (then p_len gives
        the payload's length)."""
        self.hdr = np.asarray(hdr, dtype=np.uint8)
        self.d = np.asarray(d, dtype=np.uint8).reshape(-1, 32)
        self.p = np.zeros(0, np.uint8) if p is None else np.asarray(p, dtype=np.uint8)
        self.p_len = len(self.p) if p_len is None else int(p_len)
        self.e = self.d.view(DIRENT).reshape(-1)
        self.t = self.e["t"].astype(np.int64)

    def rows(self, t: int):
        a = int(np.searchsorted(self.t, t, side="left"))
        b = int(np.searchsorted(self.t, t, side="right"))
        return a, b


def check_layout(s: HostStream, n_tensors: int, kind: int, base: int, new: int, fingerprint: int):
    """Header fields and the directory's global structure: tensors ascending,
    (tensor, chunk, kind) strictly increasing, payload offsets contiguous from
    0 and summing to the header's payload bytes.  None or an error text."""
    h = s.hdr
    u16 = lambda o: int(h[o:o + 2].view("<u2")[0])
    u32 = lambda o: int(h[o:o + 4].view("<u4")[0])
    u64 = lambda o: int(h[o:o + 8].view("<u8")[0])
    if (u32(0), u16(4), u16(6), u32(8), u32(12), u64(56)) != (0x31524344, 1, kind, 65536, 0, 0):
        return "header: magic / version / kind / chunk size / reserved"
    if (u64(16), u64(24), u64(32)) != (base, new, fingerprint):
        return "header: versions or fingerprint"
    n = len(s.e)
    if u64(40) != n or u64(48) != s.p_len:
        return f"header: {u64(40)} records / {u64(48)} bytes, stream holds {n} / {s.p_len}"
    if n == 0:
        return None
    e = s.e
    if e["t"].max() >= n_tensors:
        return "directory: tensor id out of range"
    key = (e["t"].astype(np.uint64) << np.uint64(33)) | (e["c"].astype(np.uint64) << np.uint64(1)) | \
        e["kind"].astype(np.uint64)
    if n > 1 and not (np.diff(key.astype(np.int64)) > 0).all():
        return "directory: entries not strictly ascending by (tensor, chunk, kind)"
    off, size = e["off"].astype(np.int64), e["size"].astype(np.int64)
    if off[0] != 0 or (n > 1 and not np.array_equal(off[1:], off[:-1] + size[:-1])) or \
            off[-1] + size[-1] != s.p_len:
        return "directory: payload offsets not contiguous"
    return None


def _compare_group(orc, ids, T, S, so, sn, streams, base, new, id_offset, outs):
    """Oracle encode of one group per stream kind, compared record by record;
    the oracle's streams go to outs[mode].  Returns (records, payload bytes,
    error text or None)."""
    n_rec = n_bytes = 0
    for mode, s in streams.items():
        spans = [s.rows(id_offset + t) for t in ids]
        gd = np.concatenate([s.d[a:b] for a, b in spans]) if spans else np.zeros((0, 32), np.uint8)
        ge = gd.view(DIRENT).reshape(-1)
        pay = int(ge["size"].astype(np.int64).sum())
        rc, _h, d, p = orc.encode(T, S, so, sn, mode=mode, base_version=base, new_version=new,
                                  dir_cap=32 * len(ge), payload_cap=pay)
        if rc != 0:
            return n_rec, n_bytes, f"mode {mode}, tensors {ids}: oracle returned {rc} for the GPU's sizes " \
                                   f"({len(ge)} records, {pay} bytes)"
        outs[mode] = (_h, d, p)
        od = d.reshape(-1, 32).copy()
        if len(od) != len(gd):
            return n_rec, n_bytes, f"mode {mode}, tensors {ids}: {len(gd)} GPU records, {len(od)} oracle records"
        oe = od.view(DIRENT).reshape(-1)
        o_off = oe["off"].copy()
        oe["t"] = np.asarray([id_offset + ids[int(x)] for x in oe["t"]], dtype=np.uint32)
        oe["off"] = ge["off"]
        if not np.array_equal(od, gd):
            r = int(np.nonzero((od != gd).any(1))[0][0])
            return n_rec, n_bytes, f"mode {mode}, tensors {ids}: directory entry {r} of the group differs " \
                                   f"(gpu {gd[r].tobytes().hex()} oracle {od[r].tobytes().hex()})"
        # records of one tensor are contiguous in both streams: one slice each
        r0 = 0
        for (a, b) in spans:
            n = b - a
            if n:
                g0 = int(s.e["off"][a])
                g1 = int(s.e["off"][b - 1]) + int(s.e["size"][b - 1])
                o0 = int(o_off[r0])
                if not np.array_equal(s.p[g0:g1], p[o0:o0 + (g1 - g0)]):
                    x = np.nonzero(s.p[g0:g1] != p[o0:o0 + (g1 - g0)])[0][0]
                    return n_rec, n_bytes, f"mode {mode}, tensor {id_offset + ids[0]}..: payload byte {int(x)} " \
                                           f"of its records differs"
            r0 += n
        n_rec += len(gd)
        n_bytes += pay
    return n_rec, n_bytes, None


def full_parity(orc, lay, olds, news, streams: dict, base: int, new: int, threads: int | None = None,
                id_offset: int = 0, step_check: bool = False, log=None) -> dict:
    """Compare every record of the host streams {mode: HostStream} with the
    oracle's, group by group over a thread pool.  `olds` / `news` are the
    device byte views of the layout's shards; the streams' tensor ids are the
    layout's plus `id_offset` (a window of a larger layout).  With
    step_check, each group also runs the rest of an oracle step: its
    canonical old and new tensors are gathered, the oracle's DELTA stream is
    applied to old and its RETRY stream retried over the result, which must
    equal new (the CPU baseline times this).  Returns counts, wall time and
    the first mismatch (None when every record is identical)."""
    threads = threads or host_cores()
    groups = scale_groups(lay.tensors)
    seg_index = {}
    for k, t in enumerate(lay.segments["tensor_id"]):
        seg_index.setdefault(int(t), []).append(k)
    lock = threading.Lock()
    state = {"records": 0, "bytes": 0, "groups": 0, "error": None, "canonical": 0}
    stop = threading.Event()

    def task(ids):
        if stop.is_set():
            return
        T, S, so, sn = mini_inputs(lay, ids, olds, news, seg_index)
        outs = {}
        n_rec, n_bytes, err = _compare_group(orc, ids, T, S, so, sn, streams, base, new, id_offset, outs)
        if err is None and step_check:
            err = _oracle_step(orc, ids, T, S, so, sn, outs, base, new)
        with lock:
            state["records"] += n_rec
            state["bytes"] += n_bytes
            state["groups"] += 1
            state["canonical"] += int(sum(int(x["numel"]) * int(x["elem_bytes"]) for x in T))
            if err is not None and state["error"] is None:
                state["error"] = err
                stop.set()

    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
        futs = [ex.submit(task, g) for g in groups]
        done = 0
        for f in concurrent.futures.as_completed(futs):
            f.result()
            done += 1
            if log and done % max(1, len(groups) // 8) == 0:
                log(f"oracle parity: {done}/{len(groups)} groups ({time.perf_counter() - t0:.0f}s)")
    wall = time.perf_counter() - t0
    return {"groups": state["groups"], "records": state["records"], "payload_bytes": state["bytes"],
            "canonical_bytes": state["canonical"], "identical": state["error"] is None,
            "first_mismatch": state["error"], "seconds": round(wall, 2), "threads": threads}


def _oracle_step(orc, ids, T, S, so, sn, outs, base, new):
    """The rest of one oracle step on a group: apply its DELTA stream to the
    gathered canonical old tensors, retry its RETRY stream over them; the
    result must equal the gathered new tensors.  Streams the comparison did
    not produce are encoded here."""
    for mode in (0, 1):
        if mode not in outs:
            rc, *o = orc.encode(T, S, so, sn, mode=mode, base_version=base, new_version=new)
            if rc:
                return f"tensors {ids}: oracle encode returned {rc}"
            outs[mode] = tuple(o)
    (h, d, p), (rh, rd, rp) = outs[0], outs[1]
    canon = [orc.gather(T, S, so, t) for t in range(len(T))]
    want = [orc.gather(T, S, sn, t) for t in range(len(T))]
    flags = np.zeros(max(len(d) // 32, 1), np.uint8)
    if orc.apply(T, canon, h, d, p, flags, expected_base_version=base) != 0:
        return f"tensors {ids}: oracle apply refused its own stream"
    if orc.retry(T, canon, rh, rd, rp, expected_base_version=base) != 0:
        return f"tensors {ids}: oracle retry refused its own stream"
    for t in range(len(T)):
        if not np.array_equal(canon[t], want[t]):
            return f"tensors {ids}: oracle apply + retry does not give new"
    return None
