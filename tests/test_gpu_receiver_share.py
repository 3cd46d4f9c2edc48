"""Receiver share of a 1T model on one GPU: 100 B BF16 parameters (200 GB)
plus 40 GB of uint8 NVFP4-packed tensors resident in HBM.

The DELTA stream (3 % BF16 changes, 0.085 % byte changes) is encoded window by
window (the trainer side's new values never fit beside 240 GB of receiver
state) and stitched into one stream.  The receiver is killed after 50 % of the
records; the overwrite retry stream then heals everything.  Checked: every
record of both streams byte-identical to the oracle's (window by window,
while the window's old and new values are on the device: the oracle runs per
tensor on a pool of host threads), the stitched streams' headers, order and
contiguous offsets, and every tensor equal to the new weights after the
retry (compared window by window against regenerated new values)."""
import time

import numpy as np
import pytest

from bit_exact_xor_amd import dcr, synth
from tests import stream_check

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

WINDOW_TENSORS = 256      # ~7.5 GB of new BF16 values per window


def say(*a):
    print("[case]", *a, flush=True)


def build_stream(lay, plan_full, mode, dir_buf, payload, t_old, t_new, orc=None):
    """Encode tensors window by window into one stream; returns the header.
    With the oracle given, every record of each window is compared with the
    oracle's before the window's inputs are replaced."""
    n_t = lay.n_tensors
    r_off, p_off, changed = 0, 0, 0
    checked = {"records": 0, "seconds": 0.0}
    for a in range(0, n_t, WINDOW_TENSORS):
        b = min(n_t, a + WINDOW_TENSORS)
        wl = synth.window_layout(lay, a, b)
        plan = dcr.dcr_plan_build(wl.tensors, [wl.shard_bytes(s) for s in range(wl.n_shards)], wl.segments)
        dcr.dcr_plan_upload(plan, "cuda")
        olds, news = [], []
        off = 0
        for s in range(wl.n_shards):
            nb = wl.shard_bytes(s)
            olds.append(t_old[off:off + nb])
            news.append(t_new[off:off + nb])
            off += (nb + 255) // 256 * 256
        synth.fill_shards_gpu(wl, olds, 0)
        synth.fill_shards_gpu(wl, news, 1)
        ws = dcr.workspace(plan, "cuda")
        hdr_w = torch.zeros(64, dtype=torch.uint8, device="cuda")
        res = torch.zeros(32, dtype=torch.uint8, device="cuda")
        dcr.dcr_encode(plan, olds, news, mode, 5, 6, hdr_w, dir_buf[r_off * 32:], payload[p_off:], res, ws)
        torch.cuda.synchronize()
        r = np.frombuffer(res.cpu().numpy().tobytes(), dtype=dcr.ENCODE_RESULT)[0]
        assert int(r["status"]) == 0, (a, r)
        n, pb = int(r["n_records"]), int(r["payload_bytes"])
        if orc is not None:
            hs = stream_check.HostStream(hdr_w.cpu().numpy(), dir_buf[r_off * 32:(r_off + n) * 32].cpu().numpy(),
                                         payload[p_off:p_off + pb].cpu().numpy())
            err = stream_check.check_layout(hs, wl.n_tensors, mode, 5, 6, plan.info.fingerprint)
            assert err is None, (a, err)
            pr = stream_check.full_parity(orc, wl, olds, news, {mode: hs}, 5, 6)
            assert pr["identical"], (a, pr["first_mismatch"])
            assert pr["records"] == n
            checked["records"] += n
            checked["seconds"] += pr["seconds"]
            if (a // WINDOW_TENSORS) % 8 == 0:
                say("cfg5", f"mode {mode}: tensors [{a}, {b}) identical to the oracle "
                            f"({checked['records']} records so far, {checked['seconds']:.0f} s of oracle)")
        if n:
            e32 = dir_buf[r_off * 32:(r_off + n) * 32].view(torch.int32).view(-1, 8)
            e64 = dir_buf[r_off * 32:(r_off + n) * 32].view(torch.int64).view(-1, 4)
            e32[:, 0] += a                 # tensor id within the whole layout
            e64[:, 2] += p_off             # payload offset within the whole stream
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
    if orc is not None:
        assert checked["records"] == r_off
        say("cfg5", f"mode {mode}: all {r_off} records identical to the oracle ({checked['seconds']:.0f} s)")
    return hdr, r_off, p_off, changed


def test_receiver_share_1t(orc):
    import gc
    gc.collect()
    torch.cuda.empty_cache()          # memory cached by earlier tests
    free, total = torch.cuda.mem_get_info()
    lay = synth.config5_layout()
    need = lay.total_bytes() + 2 * 8 * 10**9 + 26 * 10**9
    if free < need:
        pytest.skip(f"needs {need / 1e9:.0f} GB of free HBM, {free / 1e9:.0f} GB available")
    say("cfg5", f"{lay.n_tensors} tensors, {lay.total_bytes() / 1e9:.1f} GB resident")
    T = lay.tensors
    plan_full = dcr.dcr_plan_build(T, [lay.shard_bytes(s) for s in range(lay.n_shards)], lay.segments)
    dcr.dcr_plan_upload(plan_full, "cuda")
    sizes = [lay.shard_bytes(s) for s in range(lay.n_shards)]
    offs = np.concatenate([[0], np.cumsum([(s + 255) // 256 * 256 for s in sizes])]).astype(np.int64)
    cbuf = torch.empty(int(offs[-1]), dtype=torch.uint8, device="cuda")
    canon = [cbuf[int(offs[t]):int(offs[t]) + sizes[t]] for t in range(len(sizes))]
    synth.fill_shards_gpu(lay, canon, 0)                      # the receiver holds the base version
    wbytes = max(sum((sizes[t] + 255) // 256 * 256 for t in range(a, min(len(sizes), a + WINDOW_TENSORS)))
                 for a in range(0, len(sizes), WINDOW_TENSORS))
    t_old = torch.empty(wbytes, dtype=torch.uint8, device="cuda")
    t_new = torch.empty(wbytes, dtype=torch.uint8, device="cuda")
    ws = dcr.workspace(plan_full, "cuda")
    res = torch.zeros(32, dtype=torch.uint8, device="cuda")
    n_chunks = int(plan_full.info.n_chunks)

    # ---- DELTA stream, apply with a kill at 50 %
    dir_buf = torch.empty(32 * n_chunks, dtype=torch.uint8, device="cuda")
    payload = torch.empty(26 * 10**9, dtype=torch.uint8, device="cuda")
    t0 = time.time()
    hdr, n_rec, p_bytes, changed = build_stream(lay, plan_full, 0, dir_buf, payload, t_old, t_new, orc)
    say("cfg5", f"DELTA stream: {n_rec} records, {p_bytes / 1e9:.2f} GB, {changed} changed ({time.time() - t0:.1f}s)")
    # the stitched stream: header, order and contiguous offsets
    hs = stream_check.HostStream(hdr, dir_buf[: n_rec * 32].cpu().numpy(), None, p_len=p_bytes)
    assert stream_check.check_layout(hs, lay.n_tensors, 0, 5, 6, plan_full.info.fingerprint) is None
    del hs
    flags = torch.zeros(n_rec, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record()
    dcr.dcr_apply(plan_full, canon, hdr, dir_buf, payload, flags, 0, n_rec // 2, 5, res, ws)
    ev[1].record()
    torch.cuda.synchronize()
    ar = dcr.apply_result(res)
    assert int(ar["n_applied"]) == n_rec // 2 and int(ar["n_invalid"]) == 0
    say("cfg5", f"apply of 50 % of the records (then killed): {ev[0].elapsed_time(ev[1]):.2f} ms")
    del dir_buf, payload, flags
    torch.cuda.empty_cache()

    # ---- RETRY stream over everything
    rdir = torch.empty(32 * n_chunks, dtype=torch.uint8, device="cuda")
    rpay = torch.empty(28 * 10**9, dtype=torch.uint8, device="cuda")
    rhdr, rn, rpb, rchanged = build_stream(lay, plan_full, 1, rdir, rpay, t_old, t_new, orc)
    assert rchanged == changed and rn > 0
    hs = stream_check.HostStream(rhdr, rdir[: rn * 32].cpu().numpy(), None, p_len=rpb)
    assert stream_check.check_layout(hs, lay.n_tensors, 1, 5, 6, plan_full.info.fingerprint) is None
    del hs
    say("cfg5", f"RETRY stream: {rn} records, {rpb / 1e9:.2f} GB")
    ev[2].record()
    dcr.dcr_apply_overwrite_retry(plan_full, canon, rhdr, rdir, rpay, 5, res, ws)
    ev[3].record()
    torch.cuda.synchronize()
    ar = dcr.apply_result(res)
    assert int(ar["n_applied"]) == rn and int(ar["n_invalid"]) == 0
    say("cfg5", f"retry over all records: {ev[2].elapsed_time(ev[3]):.2f} ms")
    # every tensor equals new, window by window
    for a in range(0, lay.n_tensors, WINDOW_TENSORS):
        b = min(lay.n_tensors, a + WINDOW_TENSORS)
        wl = synth.window_layout(lay, a, b)
        news, off = [], 0
        for s in range(wl.n_shards):
            nb = wl.shard_bytes(s)
            news.append(t_new[off:off + nb])
            off += (nb + 255) // 256 * 256
        synth.fill_shards_gpu(wl, news, 1)
        for i in range(b - a):
            assert torch.equal(canon[a + i], news[i]), lay.tensor_names[a + i]
    say("cfg5", "after kill + retry: all 240 GB equal the new version")
    del cbuf, canon, rdir, rpay, t_old, t_new
    torch.cuda.empty_cache()
