"""Independent reader of the delta-stream format, for tests.

Written from the format definition alone (header, 32-byte directory entries,
16-byte-padded record sections: change bitmap (or, in the index-list layout
marked by directory byte 15, K 16-bit element indices), low byte plane, then
for 2-byte XOR records a presence bitmap + nonzero high bytes (SPARSE) or all
high bytes (DENSE); for overwrite records the upper byte planes).  It shares
nothing with the oracle or the GPU library.
"""
import numpy as np

MAGIC = 0x31524344


def pad16(x):
    return (x + 15) // 16 * 16


def header(h):
    h = np.asarray(h, dtype=np.uint8)
    u32 = lambda o: int(h[o:o + 4].view("<u4")[0])
    u64 = lambda o: int(h[o:o + 8].view("<u8")[0])
    return dict(magic=u32(0), version=int(h[4:6].view("<u2")[0]), kind=int(h[6:8].view("<u2")[0]),
                chunk_bytes=u32(8), base=u64(16), new=u64(24), fingerprint=u64(32),
                n_records=u64(40), payload_bytes=u64(48))


def dirents(d):
    d = np.asarray(d, dtype=np.uint8).reshape(-1, 32)
    out = []
    for e in d:
        out.append(dict(t=int(e[0:4].view("<u4")[0]), c=int(e[4:8].view("<u4")[0]),
                        K=int(e[8:12].view("<u4")[0]), kind=int(e[12]), hi_mode=int(e[13]),
                        w=int(e[14]), layout=int(e[15]), off=int(e[16:24].view("<u8")[0]),
                        size=int(e[24:28].view("<u4")[0]), H=int(e[28:32].view("<u4")[0])))
    return out


def decode_record(e, payload, n_c):
    """-> (indices within the chunk, payload words) of one record."""
    p = np.asarray(payload, dtype=np.uint8)[e["off"]:e["off"] + e["size"]]
    K, w = e["K"], e["w"]
    nb = (n_c + 7) // 8
    if e.get("layout", 0) == 1:
        idx = p[:2 * K].view("<u2").astype(np.int64)
        assert len(idx) == K and (np.diff(idx) > 0).all() and (idx < n_c).all()
        pos = pad16(2 * K)
    else:
        bits = np.unpackbits(p[:nb], bitorder="little")[:n_c]
        idx = np.nonzero(bits)[0]
        assert len(idx) == K
        pos = pad16(nb)
    words = p[pos:pos + K].astype(np.uint32)
    pos += pad16(K)
    if w == 2 and e["kind"] == 0:
        if e["hi_mode"] == 1:
            pres = np.unpackbits(p[pos:pos + (K + 7) // 8], bitorder="little")[:K].astype(bool)
            pos += pad16((K + 7) // 8)
            hi = np.zeros(K, dtype=np.uint32)
            hi[pres] = p[pos:pos + e["H"]]
            words |= hi << 8
        elif e["hi_mode"] == 2:
            words |= p[pos:pos + K].astype(np.uint32) << 8
    elif w >= 2:
        for b in range(1, w):
            words |= p[pos:pos + K].astype(np.uint32) << (8 * b)
            pos += pad16(K)
    return idx, words


def decode_stream(hdr, d, p, numels, widths):
    """-> list of (tensor, chunk, kind, global indices, words)."""
    out = []
    for e in dirents(d):
        E = 65536 // widths[e["t"]]
        n_c = min(E, numels[e["t"]] - e["c"] * E)
        idx, words = decode_record(e, p, n_c)
        out.append((e["t"], e["c"], e["kind"], idx + e["c"] * E, words))
    return out


def fnv1a64(data: bytes) -> int:
    h = 0xCBF29CE484222325
    for b in data:
        h ^= b
        h = (h * 0x100000001B3) & ((1 << 64) - 1)
    return h
