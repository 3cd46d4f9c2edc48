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


def hi_mode_of(K, h):
    """High-byte mode of a 2-byte XOR record with K changes, h of them with a
    nonzero high byte: NONE, SPARSE when strictly smaller than DENSE, else DENSE."""
    if h == 0:
        return 0
    return 1 if pad16((K + 7) // 8) + pad16(h) < pad16(K) else 2


def build_record(n_c, w, kind, idx, words):
    """-> (payload bytes, hi_mode, H) of one bitmap-layout record written from
    the format definition: changes idx (ascending chunk indices) carrying
    words (XOR masks or new bits)."""
    idx = [int(i) for i in idx]
    words = [int(x) for x in words]
    K = len(idx)
    out = bytearray(pad16((n_c + 7) // 8))
    for i in idx:
        out[i // 8] |= 1 << (i % 8)
    lo = bytearray(pad16(K))
    for j, x in enumerate(words):
        lo[j] = x & 0xFF
    out += lo
    if w == 1:
        return bytes(out), 0, 0
    if kind == 0:                       # XOR on 2-byte elements
        his = [(x >> 8) & 0xFF for x in words]
        h = sum(1 for b in his if b)
        mode = hi_mode_of(K, h)
        if mode == 1:
            pres = bytearray(pad16((K + 7) // 8))
            for j, b in enumerate(his):
                if b:
                    pres[j // 8] |= 1 << (j % 8)
            hp = bytearray(pad16(h))
            for q, b in enumerate(b for b in his if b):
                hp[q] = b
            out += pres + hp
            return bytes(out), 1, h
        if mode == 2:
            hp = bytearray(pad16(K))
            for j, b in enumerate(his):
                hp[j] = b
            out += hp
            return bytes(out), 2, K
        return bytes(out), 0, 0
    for b in range(1, w):               # overwrite: the upper planes
        plane = bytearray(pad16(K))
        for j, x in enumerate(words):
            plane[j] = (x >> (8 * b)) & 0xFF
        out += plane
    return bytes(out), 2, K


def build_stream(records, kind, base, new, fingerprint, numels, widths):
    """-> (header, directory, payload) as uint8 arrays for records given as
    (tensor, chunk, record kind, chunk indices, words), in the order given."""
    dirb, pay = bytearray(), bytearray()
    for (t, c, k, idx, words) in records:
        w = widths[t]
        E = 65536 // w
        n_c = min(E, numels[t] - c * E)
        body, mode, H = build_record(n_c, w, k, idx, words)
        e = bytearray(32)
        e[0:4] = int(t).to_bytes(4, "little")
        e[4:8] = int(c).to_bytes(4, "little")
        e[8:12] = len(idx).to_bytes(4, "little")
        e[12], e[13], e[14], e[15] = k, mode, w, 0
        e[16:24] = len(pay).to_bytes(8, "little")
        e[24:28] = len(body).to_bytes(4, "little")
        e[28:32] = int(H).to_bytes(4, "little")
        dirb += e
        pay += body
    h = bytearray(64)
    h[0:4] = MAGIC.to_bytes(4, "little")
    h[4:6] = (1).to_bytes(2, "little")
    h[6:8] = int(kind).to_bytes(2, "little")
    h[8:12] = (65536).to_bytes(4, "little")
    h[16:24] = int(base).to_bytes(8, "little")
    h[24:32] = int(new).to_bytes(8, "little")
    h[32:40] = int(fingerprint).to_bytes(8, "little")
    h[40:48] = (len(records)).to_bytes(8, "little")
    h[48:56] = len(pay).to_bytes(8, "little")
    as_u8 = lambda b: np.frombuffer(bytes(b), dtype=np.uint8).copy()
    return as_u8(h), as_u8(dirb), as_u8(pay)


def leb128(v):
    """Unsigned LEB128 bytes of v: seven bits per byte, low group first, the
    high bit set on every byte but the last."""
    out = bytearray()
    while True:
        b = v & 0x7F
        v >>= 7
        if v:
            out.append(b | 0x80)
        else:
            out.append(b)
            return bytes(out)


def read_gaps(sec, K):
    """-> (K indices, bytes used) from a gap section: K unsigned LEB128
    varints, gap 0 = index 0, gap j = index j - index j-1 - 1."""
    idx, pos, prev = [], 0, -1
    for _ in range(K):
        v = shift = 0
        while True:
            b = int(sec[pos])
            pos += 1
            v |= (b & 0x7F) << shift
            shift += 7
            if not b & 0x80:
                break
        prev = prev + 1 + v
        idx.append(prev)
    return np.array(idx, dtype=np.int64), pos
