"""Pipelined transfer of a stream through pinned host memory.

A pinned host buffer stands in for the network.  The sender runs
dcr_encode_pipelined and, while the encode is still going, copies each
slice it publishes device -> host on a stream of its own.  The receiver
copies each slice host -> its own device buffers on a second stream and
applies its records (dcr_apply with the slice's prefix header) on a third,
so the copy of slice k + 1 overlaps the apply of slice k.  Building and
sending overlap on the sender, receiving and patching on the receiver, and
the latency becomes about the longest leg rather than the sum (ai-feeds
summary "key modules" 5; humansand "weight teleportation" page,
"Overlapping DE and SM": the transfer into one slot runs while the bitwise
kernel works on the other).

Only copies (the copy engines) and library calls are issued here; every
step of the method runs in libdcr's kernels.
"""
import numpy as np

from . import dcr


def _u64(h: np.ndarray, off: int) -> int:
    return int(h[off:off + 8].view("<u8")[0])


class HostLoopback:
    """Pinned host staging and the receiver's device copy of a stream."""

    def __init__(self, plan: "dcr.Plan", dir_bytes: int, payload_bytes: int, device="cuda"):
        import torch
        self.plan = plan
        self.host_dir = torch.empty(max(int(dir_bytes), 32), dtype=torch.uint8, pin_memory=True)
        self.host_payload = torch.empty(max(int(payload_bytes), 16), dtype=torch.uint8, pin_memory=True)
        self.rdir = torch.empty(self.host_dir.numel(), dtype=torch.uint8, device=device)
        self.rpayload = torch.empty(self.host_payload.numel(), dtype=torch.uint8, device=device)
        self.d2h = torch.cuda.Stream(device=device)
        self.h2d = torch.cuda.Stream(device=device)
        self.apply_stream = torch.cuda.Stream(device=device)
        self.device = device

    def _fits(self, r1, p1):
        if r1 > self.host_dir.numel() // 32 or p1 > self.host_payload.numel():
            raise dcr.DcrError(dcr.DCR_E_CAPACITY, "HostLoopback", "host staging smaller than the stream")

    # ------------------------------------------------------------ sender
    def send(self, old_shards, new_shards, mode, base_version, new_version, sb: "dcr.StreamBuffers", workspace,
             n_slices: int, timeout_us: int = 30_000_000):
        """Encode with a ready watermark on the current stream; copy each
        published slice to host memory as soon as it is published.  Returns
        the prefix headers and, per slice, an event that completes when the
        slice is in host memory."""
        import torch
        # kept on the object: after a failed wait the encode may still
        # publish into it, so it must not go back to torch's pinned pool
        self._ready = ready = torch.zeros(dcr.ready_region_bytes(n_slices), dtype=torch.uint8, pin_memory=True)
        dcr.dcr_encode_pipelined(self.plan, old_shards, new_shards, mode, base_version, new_version, sb.header,
                                 sb.dir, sb.payload, sb.result, workspace, n_slices, ready)
        n = int(ready.numpy()[12:16].view("<u4")[0])
        heads, sent = [], []
        r0 = p0 = 0
        for k in range(n):
            h = dcr.dcr_ready_wait(ready, k, timeout_us)
            r1, p1 = _u64(h, 40), _u64(h, 48)
            self._fits(r1, p1)
            with torch.cuda.stream(self.d2h):
                self.host_dir[r0 * 32:r1 * 32].copy_(sb.dir[r0 * 32:r1 * 32], non_blocking=True)
                self.host_payload[p0:p1].copy_(sb.payload[p0:p1], non_blocking=True)
                ev = torch.cuda.Event()
                ev.record(self.d2h)
            heads.append(h)
            sent.append(ev)
            r0, p0 = r1, p1
        return heads, sent

    def send_serial(self, old_shards, new_shards, mode, base_version, new_version, sb: "dcr.StreamBuffers",
                    workspace):
        """The sender without pipelining: the whole encode, then the whole
        stream device -> host.  Returns the header; the caller synchronises
        the device -> host stream."""
        import torch
        dcr.dcr_encode(self.plan, old_shards, new_shards, mode, base_version, new_version, sb.header, sb.dir,
                       sb.payload, sb.result, workspace)
        torch.cuda.current_stream().synchronize()      # the host needs the stream's size
        r = sb.result_host()
        if int(r["status"]) != 0:
            raise dcr.DcrError(int(r["status"]), "HostLoopback.send_serial", "encode failed")
        n, pb = int(r["n_records"]), int(r["payload_bytes"])
        self._fits(n, pb)
        with torch.cuda.stream(self.d2h):
            self.host_dir[:n * 32].copy_(sb.dir[:n * 32], non_blocking=True)
            self.host_payload[:pb].copy_(sb.payload[:pb], non_blocking=True)
        return sb.header_host()

    # ---------------------------------------------------------- receiver
    def receive(self, heads, canon, flags, apply_workspace, base_version, sent=None):
        """Copy each slice of a stream in host memory to the receiver's
        buffers and apply its records with its prefix header, the copy of a
        slice overlapping the apply of the one before.  `sent[k]` (optional)
        is an event the copy of slice k waits for.  Returns the apply results
        (device, one per slice with records); the caller synchronises the
        apply stream."""
        import torch
        results = []
        r0 = p0 = 0
        for k, h in enumerate(heads):
            r1, p1 = _u64(h, 40), _u64(h, 48)
            self._fits(r1, p1)
            if sent is not None:
                self.h2d.wait_event(sent[k])
            with torch.cuda.stream(self.h2d):
                self.rdir[r0 * 32:r1 * 32].copy_(self.host_dir[r0 * 32:r1 * 32], non_blocking=True)
                self.rpayload[p0:p1].copy_(self.host_payload[p0:p1], non_blocking=True)
                arrived = torch.cuda.Event()
                arrived.record(self.h2d)
            if r1 > r0:
                self.apply_stream.wait_event(arrived)
                with torch.cuda.stream(self.apply_stream):
                    res = torch.empty(32, dtype=torch.uint8, device=self.device)   # the apply initialises it
                    dcr.dcr_apply(self.plan, canon, h, self.rdir, self.rpayload, flags, r0, r1 - r0, base_version,
                                  res, apply_workspace, stream=self.apply_stream)
                results.append(res)
            r0, p0 = r1, p1
        return results

    def receive_serial(self, header, canon, flags, apply_workspace, base_version):
        """The receiver without pipelining: the whole stream host -> device,
        then one apply.  Returns the apply result; the caller synchronises
        the apply stream."""
        import torch
        n, pb = _u64(header, 40), _u64(header, 48)
        self._fits(n, pb)
        with torch.cuda.stream(self.h2d):
            self.rdir[:n * 32].copy_(self.host_dir[:n * 32], non_blocking=True)
            self.rpayload[:pb].copy_(self.host_payload[:pb], non_blocking=True)
        self.h2d.synchronize()
        with torch.cuda.stream(self.apply_stream):
            res = torch.empty(32, dtype=torch.uint8, device=self.device)
            dcr.dcr_apply(self.plan, canon, header, self.rdir, self.rpayload, flags, 0, n, base_version, res,
                          apply_workspace, stream=self.apply_stream)
        return res

    # ------------------------------------------------- both on one GPU
    def run(self, old_shards, new_shards, mode, base_version, new_version, sb: "dcr.StreamBuffers", workspace,
            n_slices: int, canon, flags, apply_workspace):
        """Sender and receiver together: each slice goes device -> host ->
        device and is applied while the encode and the later slices are
        still in flight.  Returns (prefix headers, apply results)."""
        heads, sent = self.send(old_shards, new_shards, mode, base_version, new_version, sb, workspace, n_slices)
        return heads, self.receive(heads, canon, flags, apply_workspace, base_version, sent)

    def run_serial(self, old_shards, new_shards, mode, base_version, new_version, sb: "dcr.StreamBuffers",
                   workspace, canon, flags, apply_workspace):
        """Both sides one step after the other."""
        h = self.send_serial(old_shards, new_shards, mode, base_version, new_version, sb, workspace)
        self.d2h.synchronize()
        return self.receive_serial(h, canon, flags, apply_workspace, base_version)
