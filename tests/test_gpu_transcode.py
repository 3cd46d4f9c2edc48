"""GPU parity of the RETRY stream written from a DELTA stream
(dcr_encode_retry_from_delta) against the oracle's RETRY encode.

The DELTA stream fed in is the oracle's, uploaded to the device; the result
must equal the oracle's RETRY stream of the same layout byte for byte, and
applying it to old must give new.  Every test prints the case it runs before
touching the GPU.
"""
import sys

import numpy as np
import pytest

from bit_exact_xor_amd import dcr, synth
from tests import fmt, pins

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LISTS = 0x100


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gh():
    from tests import gpu_harness
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dcr.load_library()
    return gpu_harness


def dev(a, pad=16):
    """Host bytes in a device buffer of at least `pad` bytes."""
    t = torch.zeros(max(len(a), pad), dtype=torch.uint8, device="cuda")
    if len(a):
        t[: len(a)].copy_(torch.from_numpy(np.ascontiguousarray(a)))
    return t


def transcode(g, hdr, d_dev, p_dev, options=0, dir_bytes=None, payload_bytes=None):
    sb = dcr.StreamBuffers(g.plan, "cuda", dir_bytes, payload_bytes)
    dcr.dcr_encode_retry_from_delta(g.plan, g.olds, hdr, d_dev, p_dev, options, sb.header, sb.dir, sb.payload,
                                    sb.result, g.ws)
    torch.cuda.synchronize()
    return sb


def assert_same(g, sb, exp, what):
    eh, ed, ep = exp
    got = g.stream_host(sb)
    assert np.array_equal(got[0], eh), f"{what}: header differs"
    assert got[1].shape == ed.shape and np.array_equal(got[1], ed), f"{what}: directory differs"
    assert got[2].shape == ep.shape, f"{what}: payload size {got[2].shape} vs {ep.shape}"
    if not np.array_equal(got[2], ep):
        i = int(np.nonzero(got[2] != ep)[0][0])
        raise AssertionError(f"{what}: payload byte {i} differs (gpu {got[2][i]} oracle {ep[i]})")


@pytest.mark.parametrize("seed", range(24))
def test_retry_from_delta_parity(gh, orc, seed):
    """Random layouts (1-, 2- and 4-byte elements, block-scaled tensors with
    XOR and overwrite records in one chunk, transposed and split shards), at
    change rates from sparse to dense; DELTA input in the bitmap or index-list
    layout, RETRY output in either: equal to the oracle's RETRY stream, and
    applied to old it gives new."""
    rate = [None, 0.002, 0.03, 0.2][seed % 4]
    in_lists = (seed // 4) % 2 == 1
    out_lists = (seed // 8) % 2 == 1
    say("retry from delta", seed, rate, "lists in" if in_lists else "bitmap in",
        "lists out" if out_lists else "bitmap out")
    lay = synth.random_layout(1700 + seed, rate=rate, max_tensors=6, max_chunks=6.0)
    olds, news, co, cn = pins.canon_lists(lay)
    rc, dh, dd, dp = orc.encode(lay.tensors, lay.segments, olds, news, mode=LISTS if in_lists else 0,
                                base_version=7, new_version=8)
    assert rc == 0
    rc, eh, ed, ep = orc.encode(lay.tensors, lay.segments, olds, news, mode=1 | (LISTS if out_lists else 0),
                                base_version=7, new_version=8)
    assert rc == 0
    g = gh.Gpu(lay, olds, news)
    sb = transcode(g, dh, dev(dd), dev(dp), LISTS if out_lists else 0)
    assert_same(g, sb, (eh, ed, ep), f"seed {seed}")
    r = sb.result_host()
    assert int(r["n_changed"]) == int(g.encode(1).result_host()["n_changed"])
    buf, canon = g.canon_alloc(co)
    rr = g.retry(canon, sb.header_host(), sb)
    assert int(rr["n_invalid"]) == 0
    got = gh.host(canon)
    for t in range(lay.n_tensors):
        assert np.array_equal(got[t], cn[t]), (seed, t)


def test_retry_from_delta_empty_and_capacity(gh, orc):
    """No changes: an empty RETRY stream equal to the oracle's.  Buffers too
    small: status DCR_E_CAPACITY with the stream's sizes, as dcr_encode."""
    say("retry from delta: empty, capacity")
    lay = synth.random_layout(1750, max_tensors=4, max_chunks=4.0)
    olds, news, co, cn = pins.canon_lists(lay)
    rc, dh, dd, dp = orc.encode(lay.tensors, lay.segments, olds, olds, base_version=7, new_version=8)
    assert rc == 0 and len(dd) == 0
    rc, eh, ed, ep = orc.encode(lay.tensors, lay.segments, olds, olds, mode=1, base_version=7, new_version=8)
    assert rc == 0
    g = gh.Gpu(lay, olds, news)
    sb = transcode(g, dh, dev(dd), dev(dp))
    assert_same(g, sb, (eh, ed, ep), "empty")

    rc, dh, dd, dp = orc.encode(lay.tensors, lay.segments, olds, news, base_version=7, new_version=8)
    rc2, eh, ed, ep = orc.encode(lay.tensors, lay.segments, olds, news, mode=1, base_version=7, new_version=8)
    assert rc == 0 and rc2 == 0 and len(ed) > 32 and len(ep) > 16
    for dbytes, pbytes in ((32, None), (None, 16)):
        sb = transcode(g, dh, dev(dd), dev(dp), dir_bytes=dbytes, payload_bytes=pbytes)
        r = sb.result_host()
        assert int(r["status"]) == dcr.DCR_E_CAPACITY, r
        assert int(r["n_records"]) == len(ed) // 32 and int(r["payload_bytes"]) == len(ep)


def test_retry_from_delta_refused(gh, orc):
    """Host checks: a RETRY header, a short directory or payload buffer, a
    header claiming more records than two per chunk raise.  Device checks
    (status DCR_E_FORMAT, no usable stream): an entry naming a tensor the
    plan lacks, a record size that disagrees with its fields, records out of
    order (these stop the call before any record is written), a bitmap whose
    popcount is not K, a bit set in a bitmap's padding words past the
    chunk's elements (found per record, while other records are written)."""
    say("retry from delta: refused")
    lay = synth.random_layout(1751, max_tensors=6, max_chunks=8.0)
    olds, news, co, cn = pins.canon_lists(lay)
    rc, dh, dd, dp = orc.encode(lay.tensors, lay.segments, olds, news, base_version=7, new_version=8)
    assert rc == 0
    n = len(dd) // 32
    assert n > 2
    rc, rh, _rd, _rp = orc.encode(lay.tensors, lay.segments, olds, news, mode=1, base_version=7, new_version=8)
    g = gh.Gpu(lay, olds, news)
    with pytest.raises(dcr.DcrError):
        transcode(g, rh, dev(dd), dev(dp))
    with pytest.raises(dcr.DcrError):
        transcode(g, dh, dev(dd[: 32 * (n - 1)], 16), dev(dp))
    with pytest.raises(dcr.DcrError):
        transcode(g, dh, dev(dd), dev(dp[: len(dp) - 16]))

    def refused(d, p, what):
        sb = transcode(g, dh, dev(d), dev(p))
        assert int(sb.result_host()["status"]) == dcr.DCR_E_FORMAT, what

    e = dd.reshape(-1, 32)
    bad = e.copy()
    bad[0, 0:4] = np.frombuffer(np.uint32(lay.n_tensors).tobytes(), np.uint8)
    refused(bad.reshape(-1), dp, "tensor id")
    bad = e.copy()
    bad[0, 24:28] = np.frombuffer(np.uint32(int(e[0, 24:28].view("<u4")[0]) + 16).tobytes(), np.uint8)
    refused(bad.reshape(-1), dp, "record size")
    bad = e[[1, 0] + list(range(2, n))].copy()
    refused(bad.reshape(-1), dp, "order")
    # a bitmap record with a change bit cleared: popcount K - 1
    r0 = [r for r in range(n) if e[r, 15] == 0][0]
    off, size = int(e[r0, 16:24].view("<u8")[0]), int(e[r0, 24:28].view("<u4")[0])
    p = dp.copy()
    nz = int(np.nonzero(p[off:off + size])[0][0])   # inside the bitmap, which comes first
    p[off + nz] &= np.uint8(p[off + nz] - 1)
    refused(dd, p, "popcount")
    # a bit in a padding word of a bitmap (past the chunk's elements, inside
    # the 16-byte padded section): K stays right, the bit is still refused
    T = lay.tensors
    hit = False
    for r, ent in enumerate(fmt.dirents(dd)):
        w = ent["w"]
        E = 65536 // w
        n_c = min(E, int(T[ent["t"]]["numel"]) - ent["c"] * E)
        nw = (n_c + 31) // 32
        if ent["layout"] == 0 and fmt.pad16((n_c + 7) // 8) * 8 > nw * 32:
            p = dp.copy()
            p[ent["off"] + 4 * nw] |= np.uint8(1)
            refused(dd, p, f"padding bit of record {r}")
            hit = True
            break
    assert hit
    bad_h = dh.copy()
    bad_h[40:48] = np.frombuffer(np.uint64(2 * g.plan.info.n_chunks + 1).tobytes(), np.uint8)
    with pytest.raises(dcr.DcrError):
        transcode(g, bad_h, dev(np.zeros(32 * (2 * g.plan.info.n_chunks + 1), np.uint8)), dev(dp))
