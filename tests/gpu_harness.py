"""Helpers that drive libdcr.so on the GPU for the parity tests."""
import numpy as np
import torch

from bit_exact_xor_amd import dcr, synth


def shard_bytes(lay):
    return [lay.shard_bytes(s) for s in range(lay.n_shards)]


class Gpu:
    """A layout's plan, shards and workspace on the GPU."""

    def __init__(self, lay, olds=None, news=None, gen_gpu=False, device="cuda"):
        self.lay = lay
        self.device = device
        self.plan = dcr.dcr_plan_build(lay.tensors, shard_bytes(lay), lay.segments)
        dcr.dcr_plan_upload(self.plan, device)
        self.old_buf, self.olds = synth.alloc_shards(lay, device)
        self.new_buf, self.news = synth.alloc_shards(lay, device)
        if gen_gpu:
            self._hot0 = synth.fill_shards_gpu(lay, self.olds, 0)
            self._hot1 = synth.fill_shards_gpu(lay, self.news, 1)
        else:
            olds = olds if olds is not None else lay.shards_host(0)
            news = news if news is not None else lay.shards_host(1)
            for dst, src in zip(self.olds, olds):
                if dst.numel():
                    dst.copy_(torch.from_numpy(np.ascontiguousarray(src).view(np.uint8).reshape(-1)))
            for dst, src in zip(self.news, news):
                if dst.numel():
                    dst.copy_(torch.from_numpy(np.ascontiguousarray(src).view(np.uint8).reshape(-1)))
        self.ws = dcr.workspace(self.plan, device)
        torch.cuda.synchronize()

    def encode(self, mode=0, base=7, new=8, dir_bytes=None, payload_bytes=None, stage=0):
        """stage: bytes of encode staging area past the plan's workspace."""
        sb = dcr.StreamBuffers(self.plan, self.device, dir_bytes, payload_bytes)
        ws = self.ws if not stage else dcr.workspace(self.plan, self.device, stage)
        dcr.dcr_encode(self.plan, self.olds, self.news, mode, base, new, sb.header, sb.dir, sb.payload,
                       sb.result, ws)
        torch.cuda.synchronize()
        return sb

    def encode_pipelined(self, mode=0, n_slices=4, base=7, new=8, stage=0):
        """Sliced encode with a ready watermark; returns (buffers, region)."""
        sb = dcr.StreamBuffers(self.plan, self.device)
        ws = self.ws if not stage else dcr.workspace(self.plan, self.device, stage)
        ready = torch.full((dcr.ready_region_bytes(n_slices),), 0xEE, dtype=torch.uint8, pin_memory=True)
        dcr.dcr_encode_pipelined(self.plan, self.olds, self.news, mode, base, new, sb.header, sb.dir, sb.payload,
                                 sb.result, ws, n_slices, ready)
        torch.cuda.synchronize()
        return sb, ready

    def encode_retry_partial(self, delta_hdr, delta_sb, flags, base=7, new=8, stage=0):
        """Partial retry encode from a DELTA stream and its applied flags."""
        sb = dcr.StreamBuffers(self.plan, self.device)
        ws = self.ws if not stage else dcr.workspace(self.plan, self.device, stage)
        dcr.dcr_encode_retry_partial(self.plan, self.olds, self.news, delta_hdr, delta_sb.dir, flags, base, new,
                                     sb.header, sb.dir, sb.payload, sb.result, ws)
        torch.cuda.synchronize()
        return sb

    def stream_host(self, sb):
        """(header, directory, payload) bytes as numpy, trimmed to the stream."""
        r = sb.result_host()
        assert int(r["status"]) == 0, r
        n, pb = int(r["n_records"]), int(r["payload_bytes"])
        return (sb.header.cpu().numpy(), sb.dir[: n * 32].cpu().numpy(), sb.payload[:pb].cpu().numpy())

    def canon_alloc(self, init=None, align=256):
        """Canonical tensors in one device buffer, each 256-byte aligned."""
        T = self.lay.tensors
        offs, total = [], 0
        for t in range(len(T)):
            offs.append(total)
            total += (int(T[t]["numel"]) * int(T[t]["elem_bytes"]) + align - 1) // align * align
        buf = torch.zeros(max(total, align), dtype=torch.uint8, device=self.device)
        views = [buf[o:o + int(T[t]["numel"]) * int(T[t]["elem_bytes"])] for t, o in enumerate(offs)]
        if init is not None:
            for v, x in zip(views, init):
                if v.numel():
                    v.copy_(torch.from_numpy(np.ascontiguousarray(x).view(np.uint8).reshape(-1)))
        return buf, views

    def apply(self, canon, hdr, sb, flags, first=0, n=None, base=7):
        nrec = int(hdr[40:48].view("<u8")[0])
        n = nrec - first if n is None else n
        res = torch.zeros(32, dtype=torch.uint8, device=self.device)
        dcr.dcr_apply(self.plan, canon, hdr, sb.dir, sb.payload, flags, first, n, base, res, self.ws)
        torch.cuda.synchronize()
        return dcr.apply_result(res)

    def retry(self, canon, hdr, sb, base=7):
        res = torch.zeros(32, dtype=torch.uint8, device=self.device)
        dcr.dcr_apply_overwrite_retry(self.plan, canon, hdr, sb.dir, sb.payload, base, res, self.ws)
        torch.cuda.synchronize()
        return dcr.apply_result(res)


def chunk_starts(lay):
    """Plan index of each tensor's first chunk (tensor order, 64 KiB chunks)."""
    n = [(int(t["numel"]) * int(t["elem_bytes"]) + 65535) // 65536 for t in lay.tensors]
    return np.concatenate([[0], np.cumsum(n)]).astype(np.int64)


def expected_prefixes(lay, dir_bytes, payload_total, n_slices):
    """(records, payload bytes) of the stream cut after each slice of a
    pipelined encode, from a finished stream's directory and the slice rule
    (slice k ends at chunk 256 * floor((k + 1) * nb / n), nb = fix-up blocks)."""
    starts = chunk_starts(lay)
    nch = int(starts[-1])
    nb = (nch + 255) // 256
    n = min(n_slices, max(nb, 1))
    d = np.asarray(dir_bytes, dtype=np.uint8).reshape(-1, 32)
    t = d[:, 0:4].copy().view("<u4").ravel().astype(np.int64)
    c = d[:, 4:8].copy().view("<u4").ravel().astype(np.int64)
    off = d[:, 16:24].copy().view("<u8").ravel().astype(np.int64)
    g = starts[t] + c
    assert (np.diff(g) >= 0).all()
    out = []
    for k in range(n):
        end = min(256 * ((k + 1) * nb // n), nch)
        r = int(np.searchsorted(g, end, side="left"))
        out.append((r, int(off[r]) if r < len(g) else int(payload_total)))
    return n, out


def scatter_shards(lay, canon, device="cuda", fill=0xA5):
    """Receiver shards of layout `lay` holding the canonical tensors `canon`."""
    return synth.scatter_canonical_gpu(lay, canon, device, fill)


def host(views):
    return [v.cpu().numpy() for v in views]
