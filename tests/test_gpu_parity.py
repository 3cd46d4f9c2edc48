"""GPU parity: libdcr.so (gfx950 kernels) against the CPU oracle.

Stream bytes (header, directory, payload) must equal the oracle's byte for
byte, and patched weights must equal the oracle's (= the new weights) bit for
bit.  Every test prints the case it runs before touching the GPU.
"""
import sys

import numpy as np
import pytest

from bit_exact_xor_amd import dcr, synth
from tests import fmt, pins

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gh():
    from tests import gpu_harness
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dcr.load_library()
    return gpu_harness


def oracle_stream(orc, lay, olds, news, mode=0):
    rc, h, d, p = orc.encode(lay.tensors, lay.segments, olds, news, mode=mode, base_version=7, new_version=8)
    assert rc == 0
    return h, d, p


def assert_same_stream(got, exp, what=""):
    gh_, gd, gp = got
    eh, ed, ep = exp
    assert np.array_equal(gh_, eh), f"{what}: header differs"
    assert gd.shape == ed.shape, f"{what}: directory size {gd.shape} vs {ed.shape}"
    if not np.array_equal(gd, ed):
        bad = np.nonzero((gd.reshape(-1, 32) != ed.reshape(-1, 32)).any(1))[0]
        r = int(bad[0])
        raise AssertionError(f"{what}: directory entry {r} differs: gpu {fmt.dirents(gd[r*32:r*32+32])} "
                             f"oracle {fmt.dirents(ed[r*32:r*32+32])}")
    assert gp.shape == ep.shape, f"{what}: payload size {gp.shape} vs {ep.shape}"
    if not np.array_equal(gp, ep):
        i = int(np.nonzero(gp != ep)[0][0])
        ents = fmt.dirents(ed)
        rec = [e for e in ents if e["off"] <= i < e["off"] + e["size"]]
        raise AssertionError(f"{what}: payload byte {i} differs (gpu {gp[i]} oracle {ep[i]}) in {rec}")


SEEDS = list(range(40))


def stage_sizes(g):
    """Staging areas: none, too small (both run in-order look-back), and one
    holding every chunk's slot (no chunk waits)."""
    full = int(g.plan.info.max_payload_bytes)
    return (0, full // 2, full)


@pytest.mark.parametrize("seed", SEEDS)
def test_random_layout_parity(gh, orc, seed):
    """Random layouts: 1/2/4-byte elements, all routes, split / transposed
    shards, ragged tails, empty tensors."""
    say("random layout", seed)
    lay = synth.random_layout(seed)
    olds, news, co, cn = pins.canon_lists(lay)
    g = gh.Gpu(lay, olds, news)
    for mode in (0, 1):
        exp = oracle_stream(orc, lay, olds, news, mode)
        for stage in stage_sizes(g):
            sb = g.encode(mode, stage=stage)
            assert_same_stream(g.stream_host(sb), exp, f"seed {seed} mode {mode} stage {stage}")
    sb = g.encode(0)
    hdr, d, p = g.stream_host(sb)
    n = len(d) // 32
    buf, canon = g.canon_alloc(co)
    flags = torch.zeros(max(n, 1), dtype=torch.uint8, device="cuda")
    r = g.apply(canon, hdr, sb, flags)
    assert int(r["n_applied"]) == n and int(r["n_invalid"]) == 0
    got = gh.host(canon)
    for t in range(lay.n_tensors):
        assert np.array_equal(got[t], cn[t]), (seed, t)
    assert bool((flags[:n] == 1).all()) if n else True


def test_no_changes(gh, orc):
    """Degenerate inputs: new equal to old (every chunk scanned, no record
    written) and a plan whose tensors are all empty (no chunk at all): both
    stream kinds, every staging area, equal to the oracle's empty streams;
    the empty DELTA stream applied and the empty RETRY stream retried leave
    the weights as they were."""
    lay = synth.random_layout(2400, max_tensors=5, max_chunks=4.0)
    olds, news, co, cn = pins.canon_lists(lay)
    b = synth._Builder("empty", 1)
    b.tensor("e0", 0, 2)
    b.tensor("e1", 0, 1)
    b.shard(0, 2)
    empty = b.build()
    empty.values = ([np.zeros(0, np.uint16)], [np.zeros(0, np.uint16)])
    cases = (("new = old", lay, olds, co), ("empty plan", empty, empty.values[0], [np.zeros(0, np.uint8)] * 2))
    for name, L, o, c0 in cases:
        say("no changes:", name)
        g = gh.Gpu(L, o, o)
        for mode in (0, 1):
            exp = oracle_stream(orc, L, o, o, mode)
            assert len(exp[1]) == 0 and len(exp[2]) == 0
            for stage in stage_sizes(g):
                sb = g.encode(mode, stage=stage)
                assert_same_stream(g.stream_host(sb), exp, f"{name} mode {mode} stage {stage}")
            hdr = sb.header.cpu().numpy()
            buf, canon = g.canon_alloc(c0)
            if mode == 0:
                r = g.apply(canon, hdr, sb, torch.zeros(1, dtype=torch.uint8, device="cuda"))
            else:
                r = g.retry(canon, hdr, sb)
            assert int(r["n_applied"]) == 0 and int(r["n_invalid"]) == 0 and int(r["n_skipped"]) == 0, r
            got = gh.host(canon)
            for t in range(L.n_tensors):
                assert np.array_equal(got[t], c0[t]), (name, mode, t)


@pytest.mark.parametrize("rate", (None, 0.7))
@pytest.mark.parametrize("ws", range(1, 8))
def test_width_set_parity(gh, orc, ws, rate):
    """The in-order encode has one build per set of element widths a plan
    holds: a layout of each set (1-, 2- and 4-byte tensors), at its own
    change rate and at 70 % (records over several LDS windows), both stream
    kinds, with no staging area, a small one and a full one, against the
    oracle; the DELTA stream applied and the RETRY stream retried give new."""
    say("width set", ws, "rate", rate)
    lay = synth.width_set_layout(ws, rate=rate)
    olds, news, co, cn = pins.canon_lists(lay)
    g = gh.Gpu(lay, olds, news)
    for mode in (0, 1):
        exp = oracle_stream(orc, lay, olds, news, mode)
        for stage in stage_sizes(g):
            sb = g.encode(mode, stage=stage)
            assert_same_stream(g.stream_host(sb), exp, f"width set {ws} mode {mode} stage {stage}")
        hdr, d, p = g.stream_host(sb)
        n = len(d) // 32
        buf, canon = g.canon_alloc(co)
        if mode == 0:
            flags = torch.zeros(max(n, 1), dtype=torch.uint8, device="cuda")
            r = g.apply(canon, hdr, sb, flags)
        else:
            r = g.retry(canon, hdr, sb)
        assert int(r["n_applied"]) == n and int(r["n_invalid"]) == 0, r
        got = gh.host(canon)
        for t in range(lay.n_tensors):
            assert np.array_equal(got[t], cn[t]), (ws, mode, t)


@pytest.mark.parametrize("seed", range(6))
def test_dedup_involution_retry(gh, orc, seed):
    """Duplicates are skipped; a XOR stream applied twice restores old; the
    overwrite retry heals half-applied, torn and duplicated states."""
    say("dedup / involution / retry", seed)
    lay = synth.random_layout(600 + seed)
    olds, news, co, cn = pins.canon_lists(lay)
    g = gh.Gpu(lay, olds, news)
    sb = g.encode(0)
    hdr, d, p = g.stream_host(sb)
    n = len(d) // 32
    buf, canon = g.canon_alloc(co)
    flags = torch.zeros(max(n, 1), dtype=torch.uint8, device="cuda")
    g.apply(canon, hdr, sb, flags, 0, n // 2)                 # killed at 50 %
    r = g.apply(canon, hdr, sb, flags)                        # resume: first half skipped
    assert int(r["n_skipped"]) == n // 2 and int(r["n_applied"]) == n - n // 2
    got = gh.host(canon)
    for t in range(lay.n_tensors):
        assert np.array_equal(got[t], cn[t])
    # XOR-only twice restores old
    xor_only = all(e["kind"] == 0 for e in fmt.dirents(d))
    if xor_only and n:
        flags.zero_()
        g.apply(canon, hdr, sb, flags)
        got = gh.host(canon)
        for t in range(lay.n_tensors):
            assert np.array_equal(got[t], co[t])
    # retry from several prior states built by the oracle on the host
    rsb = g.encode(1)
    rh, rd, rp = g.stream_host(rsb)
    states = [[x.copy() for x in co]]
    W = [x.copy() for x in co]
    f = np.zeros(max(n, 1), np.uint8)
    orc.apply(lay.tensors, W, hdr, d, p, f, 0, n // 2, expected_base_version=7)
    states.append(W)
    if n:
        W = [x.copy() for x in co]
        orc.apply_record_part(lay.tensors, W, d, p, n // 2, 0, max(fmt.dirents(d)[n // 2]["K"] // 2, 1))
        states.append(W)
        W = [x.copy() for x in co]
        f = np.zeros(n, np.uint8)
        orc.apply(lay.tensors, W, hdr, d, p, f, expected_base_version=7)
        f[::2] = 0
        orc.apply(lay.tensors, W, hdr, d, p, f, expected_base_version=7)
        states.append(W)
    for si, st in enumerate(states):
        buf, canon = g.canon_alloc(st)
        g.retry(canon, rh, rsb)
        once = gh.host(canon)
        g.retry(canon, rh, rsb)
        twice = gh.host(canon)
        for t in range(lay.n_tensors):
            assert np.array_equal(once[t], cn[t]), (si, t)
            assert np.array_equal(twice[t], cn[t]), (si, t)


def test_config1_parity(gh, orc):
    """Config 1: one 4096x4096 BF16 tensor, 1 % changed + 64 forced +-0 flips."""
    say("config 1")
    lay = synth.config1_layout()
    old, new, _lr, pos = synth.config1_values(lay, lr=synth.CFG1_LR)
    g = gh.Gpu(lay, [old], [new])
    exp = oracle_stream(orc, lay, [old], [new])
    for stage in stage_sizes(g):
        assert_same_stream(g.stream_host(g.encode(0, stage=stage)), exp, f"config 1 stage {stage}")
    sb = g.encode(0)
    got = g.stream_host(sb)
    assert int(sb.result_host()["n_changed"]) == int(np.count_nonzero(old != new))
    buf, canon = g.canon_alloc([old])
    flags = torch.zeros(len(got[1]) // 32, dtype=torch.uint8, device="cuda")
    g.apply(canon, got[0], sb, flags)
    assert np.array_equal(canon[0].cpu().numpy().view(np.uint16), new)
    for mode in (1,):
        assert_same_stream(g.stream_host(g.encode(mode)), oracle_stream(orc, lay, [old], [new], mode), "cfg1 retry")


def test_llama_small_gpu_generated(gh, orc):
    """Scaled-down TP=4 Llama layout with shards generated on the GPU: the
    GPU generator reproduces the numpy one, and the streams match."""
    say("llama small, gpu-generated shards")
    lay = synth.llama_layout(hidden=256, layers=2, ffn=640, n_q=8, n_kv=4, head_dim=32, vocab=1000, tp=4,
                             rate=0.03)
    g = gh.Gpu(lay, gen_gpu=True)
    olds, news = lay.shards_host(0), lay.shards_host(1)
    for s in range(lay.n_shards):
        assert np.array_equal(g.olds[s].cpu().numpy(), olds[s].view(np.uint8)), s
        assert np.array_equal(g.news[s].cpu().numpy(), news[s].view(np.uint8)), s
    for mode in (0, 1):
        exp = oracle_stream(orc, lay, olds, news, mode)
        for stage in stage_sizes(g):
            assert_same_stream(g.stream_host(g.encode(mode, stage=stage)), exp, f"llama small mode {mode} {stage}")


def test_determinism(gh):
    """Ten encodes of the same input give identical bytes (look-back order
    varies from run to run; the stream may not)."""
    say("determinism")
    lay = synth.llama_layout(hidden=256, layers=2, ffn=640, n_q=8, n_kv=4, head_dim=32, vocab=1000, tp=4,
                             rate=0.05)
    g = gh.Gpu(lay, gen_gpu=True)
    ref = g.stream_host(g.encode(0))
    for i in range(10):
        got = g.stream_host(g.encode(0, stage=stage_sizes(g)[i % 3]))
        for a, b in zip(got, ref):
            assert np.array_equal(a, b)


@pytest.mark.parametrize("seed,rate", [(31, None), (7, 0.2)])
def test_dense_records_repeated(gh, orc, seed, rate):
    """Dense chunks whose records span several LDS output windows (1-byte
    overwrite records near 20 % change, 2-byte XOR records): twelve staged and
    four in-order encodes of the same input all equal the oracle's stream."""
    say("dense records repeated", seed)
    lay = synth.random_layout(seed, rate=rate)
    olds, news, _co, _cn = pins.canon_lists(lay)
    g = gh.Gpu(lay, olds, news)
    exp = oracle_stream(orc, lay, olds, news, 0)
    full = stage_sizes(g)[2]
    for i in range(16):
        stage = full if i < 12 else 0
        assert_same_stream(g.stream_host(g.encode(0, stage=stage)), exp, f"dense seed {seed} run {i} stage {stage}")


@pytest.mark.parametrize("seed", range(8))
def test_retry_partial(gh, orc, seed):
    """Partial retry after a kill at 0 %, 50 % and 100 % of the records: the
    stream equals the oracle's byte for byte (staged, in order and with a
    too-small staging area) and applying it heals the receiver to new."""
    say("partial retry", seed)
    lay = synth.random_layout(1000 + seed, max_tensors=6, max_chunks=8.0)
    olds, news, co, cn = pins.canon_lists(lay)
    g = gh.Gpu(lay, olds, news)
    sb = g.encode(0)
    hdr, d, _p = g.stream_host(sb)
    n = len(d) // 32
    for k in sorted({0, n // 2, n}):
        buf, canon = g.canon_alloc(co)
        flags = torch.zeros(max(n, 1), dtype=torch.uint8, device="cuda")
        if k:
            g.apply(canon, hdr, sb, flags, 0, k)
        fh = flags.cpu().numpy()
        rc, eh, ed, ep = orc.encode_retry_partial(lay.tensors, lay.segments, olds, news, hdr, d, fh,
                                                   base_version=7, new_version=8)
        assert rc == 0
        for stage in stage_sizes(g):
            psb = g.encode_retry_partial(hdr, sb, flags, stage=stage)
            assert_same_stream(g.stream_host(psb), (eh, ed, ep), f"partial seed {seed} kill {k} stage {stage}")
        ph = g.stream_host(psb)[0]
        r = g.retry(canon, ph, psb)
        assert int(r["n_invalid"]) == 0
        got = gh.host(canon)
        for t in range(lay.n_tensors):
            assert np.array_equal(got[t], cn[t]), (seed, k, t)


def test_retry_partial_refused(gh):
    """Partial retry refuses a RETRY header (host check), a short directory
    buffer, and (on the device) an entry naming a tensor the plan lacks."""
    say("partial retry refused")
    lay = synth.random_layout(1001, max_tensors=6, max_chunks=8.0)
    g = gh.Gpu(lay)
    sb = g.encode(0)
    hdr, d, _p = g.stream_host(sb)
    n = len(d) // 32
    flags = torch.zeros(max(n, 1), dtype=torch.uint8, device="cuda")
    rsb = g.encode(1)
    with pytest.raises(dcr.DcrError):
        g.encode_retry_partial(rsb.header.cpu().numpy(), sb, flags)
    assert n > 1
    short = type("S", (), {"dir": sb.dir[: 32 * (n - 1)]})()
    with pytest.raises(dcr.DcrError):
        g.encode_retry_partial(hdr, short, flags)
    bad = sb.dir.clone()
    bad[0:4] = torch.tensor(list(np.uint32(lay.n_tensors).tobytes()), dtype=torch.uint8, device="cuda")
    bsb = type("S", (), {"dir": bad})()
    psb = g.encode_retry_partial(hdr, bsb, flags)
    assert int(psb.result_host()["status"]) == dcr.DCR_E_FORMAT


@pytest.mark.parametrize("seed", range(12))
def test_index_lists_parity(gh, orc, seed):
    """Index-list layout (encode option): DELTA and RETRY streams equal the
    oracle's byte for byte with every staging mode, at change rates that put
    list records in one LDS window and across several; applying them gives
    new, from old and from a kill at 50 % through the RETRY stream."""
    rate = [0.002, 0.03, 0.05, 0.2][seed % 4]
    say("index lists", seed, rate)
    lay = synth.random_layout(1300 + seed, rate=rate, max_tensors=5, max_chunks=6.0)
    olds, news, co, cn = pins.canon_lists(lay)
    g = gh.Gpu(lay, olds, news)
    streams = {}
    for mode in (0, 1):
        rc, eh, ed, ep = orc.encode(lay.tensors, lay.segments, olds, news, mode=mode | 0x100,
                                    base_version=7, new_version=8)
        assert rc == 0
        for stage in stage_sizes(g):
            sb = g.encode(mode | dcr.ENC_INDEX_LISTS, stage=stage)
            assert_same_stream(g.stream_host(sb), (eh, ed, ep), f"lists seed {seed} mode {mode} stage {stage}")
        streams[mode] = sb
    hdr, d, _p = g.stream_host(streams[0])
    n = len(d) // 32
    buf, canon = g.canon_alloc(co)
    flags = torch.zeros(max(n, 1), dtype=torch.uint8, device="cuda")
    r = g.apply(canon, hdr, streams[0], flags)
    assert int(r["n_applied"]) == n and int(r["n_invalid"]) == 0
    got = gh.host(canon)
    for t in range(lay.n_tensors):
        assert np.array_equal(got[t], cn[t]), (seed, t)
    buf, canon = g.canon_alloc(co)
    flags.zero_()
    g.apply(canon, hdr, streams[0], flags, 0, n // 2)
    rh = g.stream_host(streams[1])[0]
    r = g.retry(canon, rh, streams[1])
    assert int(r["n_invalid"]) == 0
    got = gh.host(canon)
    for t in range(lay.n_tensors):
        assert np.array_equal(got[t], cn[t]), (seed, t)


def test_index_lists_corrupt_refused(gh):
    """A list record whose indices do not ascend strictly (two swapped, or
    one repeated) is refused before any write."""
    say("index lists corrupt")
    lay = synth.random_layout(1301, rate=0.03, max_tensors=5, max_chunks=6.0)
    olds, news, co, cn = pins.canon_lists(lay)
    g = gh.Gpu(lay, olds, news)
    sb = g.encode(dcr.ENC_INDEX_LISTS)
    hdr, d, p = g.stream_host(sb)
    ents = fmt.dirents(d)
    li = [i for i, e in enumerate(ents) if e["layout"] == 1 and e["K"] >= 2]
    assert li
    e = ents[li[0]]
    for how in ("swap", "repeat"):
        bad = sb.payload.clone()
        o = e["off"]
        if how == "swap":
            bad[o:o + 2], bad[o + 2:o + 4] = sb.payload[o + 2:o + 4].clone(), sb.payload[o:o + 2].clone()
        else:
            last = o + 2 * (e["K"] - 1)
            bad[last:last + 2] = sb.payload[last - 2:last].clone()
        bsb = type("S", (), {"dir": sb.dir, "payload": bad})()
        buf, canon = g.canon_alloc(co)
        flags = torch.zeros(len(ents), dtype=torch.uint8, device="cuda")
        r = g.apply(canon, hdr, bsb, flags, li[0], 1)
        assert int(r["n_invalid"]) == 1 and int(r["first_invalid"]) == li[0], how
        got = gh.host(canon)
        for t in range(lay.n_tensors):
            assert np.array_equal(got[t], co[t]), how


@pytest.mark.parametrize("seed", range(10))
@pytest.mark.parametrize("lists", [False, True], ids=["bitmap", "lists"])
def test_apply_sharded(gh, orc, seed, lists):
    """Apply into a receiver's own layout (random pieces at unaligned cuts,
    reversed blocks, transposed storage, gaps between placements): the
    receiver shards end byte-identical to the new tensors scattered into that
    layout, gaps untouched, and the oracle's gather of them gives new; also
    after a kill at 50 % and the overwrite retry into the same layout."""
    say("apply sharded", seed, "lists" if lists else "bitmap")
    lay = synth.random_layout(1400 + seed, max_tensors=5, max_chunks=6.0)
    lay_r = synth.receiver_layout(lay, 77 + seed)
    olds, news, co, cn = pins.canon_lists(lay)
    g = gh.Gpu(lay, olds, news)
    opt = dcr.ENC_INDEX_LISTS if lists else 0
    sb = g.encode(opt)
    hdr, d, _p = g.stream_host(sb)
    n = len(d) // 32
    rplan = dcr.dcr_plan_build(lay_r.tensors, [lay_r.shard_bytes(s) for s in range(lay_r.n_shards)],
                               lay_r.segments)
    dcr.dcr_plan_upload(rplan, "cuda")
    ws = dcr.workspace(rplan, "cuda")
    exp_buf, exp_sh = gh.scatter_shards(lay_r, cn)
    eh = [x.cpu().numpy() for x in exp_sh]
    for t in range(lay.n_tensors):   # the scatter is the receiver layout: the oracle's gather reads new back
        assert np.array_equal(orc.gather(lay_r.tensors, lay_r.segments, eh, t), cn[t]), (seed, t)
    res = torch.zeros(32, dtype=torch.uint8, device="cuda")
    rbuf, rsh = gh.scatter_shards(lay_r, co)
    flags = torch.zeros(max(n, 1), dtype=torch.uint8, device="cuda")
    dcr.dcr_apply_sharded(rplan, rsh, hdr, sb.dir, sb.payload, flags, 0, n, 7, res, ws)
    torch.cuda.synchronize()
    r = dcr.apply_result(res)
    assert int(r["n_applied"]) == n and int(r["n_invalid"]) == 0
    assert torch.equal(rbuf, exp_buf), seed
    # kill at 50 %, then the RETRY stream into the same layout
    rbuf, rsh = gh.scatter_shards(lay_r, co)
    flags.zero_()
    dcr.dcr_apply_sharded(rplan, rsh, hdr, sb.dir, sb.payload, flags, 0, n // 2, 7, res, ws)
    rsb = g.encode(1 | opt)
    rh = g.stream_host(rsb)[0]
    dcr.dcr_apply_overwrite_retry_sharded(rplan, rsh, rh, rsb.dir, rsb.payload, 7, res, ws)
    torch.cuda.synchronize()
    assert int(dcr.apply_result(res)["n_invalid"]) == 0
    assert torch.equal(rbuf, exp_buf), seed


def test_apply_sharded_gate_up_interleaved(gh, orc):
    """A receiver engine that stores each rank's fused gate/up weight with
    gate and up rows interleaved in groups of 64 (the physical layout of the
    humansand "weight teleportation" page, "Working with low-precision RL"),
    sharded TP=4: the DELTA stream of a TP=4 trainer applied straight into
    it, and a kill at 50 % healed by the RETRY stream; the receiver shards
    end byte-identical to the new tensors scattered into the layout (the
    scatter checked by the oracle's gather), and the layout's own assembly
    (select every other 64-row group) reads new back."""
    kw = dict(hidden=256, layers=2, ffn=1024, n_q=8, n_kv=4, head_dim=32, vocab=1000, tp=4, rate=0.03)
    say("apply sharded, gate/up interleaved in 64-row groups")
    lay = synth.llama_layout(**kw)
    lay_r = synth.llama_layout(**kw, gate_up_group=64)
    olds, news = lay.shards_host(0), lay.shards_host(1)
    # this layout assembles with torch ops: canonical tensors from the host shards
    co, cn = ([x.reshape(-1).numpy().view(np.uint8).copy()
               for x in lay.assemble([torch.from_numpy(np.ascontiguousarray(v).view(np.int16)) for v in vs])]
              for vs in (olds, news))
    g = gh.Gpu(lay, olds, news)
    sb = g.encode(0)
    hdr, d, _p = g.stream_host(sb)
    n = len(d) // 32
    rplan = dcr.dcr_plan_build(lay_r.tensors, [lay_r.shard_bytes(s) for s in range(lay_r.n_shards)],
                               lay_r.segments)
    dcr.dcr_plan_upload(rplan, "cuda")
    assert rplan.info.fingerprint == g.plan.info.fingerprint
    ws = dcr.workspace(rplan, "cuda")
    exp_buf, exp_sh = gh.scatter_shards(lay_r, cn)
    eh = [x.cpu().numpy() for x in exp_sh]
    for t in range(lay.n_tensors):
        assert np.array_equal(orc.gather(lay_r.tensors, lay_r.segments, eh, t), cn[t]), t
    res = torch.zeros(32, dtype=torch.uint8, device="cuda")
    flags = torch.zeros(max(n, 1), dtype=torch.uint8, device="cuda")
    rbuf, rsh = gh.scatter_shards(lay_r, co)
    dcr.dcr_apply_sharded(rplan, rsh, hdr, sb.dir, sb.payload, flags, 0, n, 7, res, ws)
    torch.cuda.synchronize()
    r = dcr.apply_result(res)
    assert int(r["n_applied"]) == n and int(r["n_invalid"]) == 0
    assert torch.equal(rbuf, exp_buf)
    got = lay_r.assemble([x.view(torch.int16) for x in rsh])
    for t in range(lay.n_tensors):
        assert np.array_equal(got[t].reshape(-1).cpu().numpy().view(np.uint8), cn[t]), lay.tensor_names[t]
    rbuf, rsh = gh.scatter_shards(lay_r, co)
    flags.zero_()
    dcr.dcr_apply_sharded(rplan, rsh, hdr, sb.dir, sb.payload, flags, 0, n // 2, 7, res, ws)
    rsb = g.encode(1)
    rh = g.stream_host(rsb)[0]
    dcr.dcr_apply_overwrite_retry_sharded(rplan, rsh, rh, rsb.dir, rsb.payload, 7, res, ws)
    torch.cuda.synchronize()
    assert int(dcr.apply_result(res)["n_invalid"]) == 0
    assert torch.equal(rbuf, exp_buf)


def test_apply_sharded_refuses_overlapping_layout(gh):
    """A receiver layout that maps two canonical elements to one shard
    element cannot be applied into."""
    say("apply sharded, overlapping layout")
    lay = synth.random_layout(1401, max_tensors=5, max_chunks=6.0)
    T = lay.tensors[:1].copy()
    n = int(T[0]["numel"])
    assert n >= 2
    S = np.zeros(2, dtype=synth.SEGMENT_DT)
    for i, (c0, c1) in enumerate(((0, n // 2), (n // 2, n))):
        S[i]["tensor_id"], S[i]["shard_id"], S[i]["ndim"] = 0, 0, 1
        S[i]["shard_off"], S[i]["canon_off"] = 0, c0          # both halves at shard offset 0
        S[i]["extent"] = [c1 - c0, 1, 1, 1]
        S[i]["shard_stride"] = [1, 0, 0, 0]
        S[i]["canon_stride"] = [1, 0, 0, 0]
    rplan = dcr.dcr_plan_build(T, [n * int(T[0]["elem_bytes"])], S)
    dcr.dcr_plan_upload(rplan, "cuda")
    shard = torch.zeros(n * int(T[0]["elem_bytes"]), dtype=torch.uint8, device="cuda")
    hdr = np.zeros(64, dtype=np.uint8)
    hdr[0:4] = np.frombuffer(np.uint32(0x31524344).tobytes(), np.uint8)
    hdr[4:6] = np.frombuffer(np.uint16(1).tobytes(), np.uint8)
    hdr[8:12] = np.frombuffer(np.uint32(65536).tobytes(), np.uint8)
    hdr[32:40] = np.frombuffer(np.uint64(rplan.info.fingerprint).tobytes(), np.uint8)
    res = torch.zeros(32, dtype=torch.uint8, device="cuda")
    flags = torch.zeros(1, dtype=torch.uint8, device="cuda")
    dbuf = torch.zeros(32, dtype=torch.uint8, device="cuda")
    with pytest.raises(dcr.DcrError):
        dcr.dcr_apply_sharded(rplan, [shard], hdr, dbuf, dbuf, flags, 0, 0, 0, res, dcr.workspace(rplan, "cuda"))


PIPE_CASES = [("random", 0), ("random", 4), ("random", 6), ("llama", 0), ("moe", 0)]


def pipe_layout(kind, seed):
    if kind == "random":
        # 700-1200 chunks of all widths and routes: several fix-up blocks
        return synth.random_layout(seed, max_tensors=24, max_chunks=120.0)
    if kind == "llama":
        return synth.llama_layout(hidden=1024, layers=4, ffn=2816, n_q=16, n_kv=4, head_dim=64, vocab=8000, tp=4,
                                  rate=0.03)
    # block-scaled experts with fp32 scale tensors
    return synth.moe_layout(hidden=512, layers=2, n_exp=16, moe_ffn=256, n_q=8, n_kv=2, head_dim=64, vocab=4000,
                            ep=4, rate=0.05, variant="hot")


def pipe_canon(kind, lay):
    """Host shards and canonical old / new (uint8) of a pipelined-encode case;
    the model layouts assemble their tensors with torch ops."""
    if kind == "random":
        return pins.canon_lists(lay)
    olds, news = lay.shards_host(0), lay.shards_host(1)
    typed_t = {1: np.uint8, 2: np.int16, 4: np.int32}

    def canon(xs):
        ts = [torch.from_numpy(np.ascontiguousarray(x).view(typed_t[x.dtype.itemsize])) for x in xs]
        return [t.reshape(-1).contiguous().view(torch.uint8).numpy().copy() for t in lay.assemble(ts)]
    return olds, news, canon(olds), canon(news)


@pytest.mark.parametrize("kind,seed", PIPE_CASES)
def test_pipelined_encode(gh, orc, kind, seed):
    """Sliced encode with a ready watermark (in-order and staged, DELTA and
    RETRY, with and without index lists): the stream equals the oracle's; every
    slice is published; prefix header k is the final header with the records
    and payload bytes of the chunks before slice k's end; applying each
    prefix's new records with its own header, slice by slice, gives new."""
    say("pipelined encode", kind, seed)
    lay = pipe_layout(kind, seed)
    olds, news, co, cn = pipe_canon(kind, lay)
    g = gh.Gpu(lay, olds, news)
    starts = gh.chunk_starts(lay)
    say("pipelined encode", kind, seed, f"{int(starts[-1])} chunks")
    for mode in (0, 1, dcr.ENC_INDEX_LISTS):
        exp = oracle_stream(orc, lay, olds, news, mode)
        for stage in (0, int(g.plan.info.max_payload_bytes)):
            for n_slices in (1, 3, 1000):
                what = f"{kind} {seed} mode {mode} stage {stage} slices {n_slices}"
                sb, ready = g.encode_pipelined(mode, n_slices, stage=stage)
                got = g.stream_host(sb)
                assert_same_stream(got, exp, what)
                rg = ready.numpy()
                n, pre = gh.expected_prefixes(lay, exp[1], len(exp[2]), n_slices)
                assert int(rg[12:16].view("<u4")[0]) == n, what
                assert int(rg[0:8].view("<u8")[0]) == n and int(rg[8:12].view("<i4")[0]) == 0, what
                for k, (r, pb) in enumerate(pre):
                    h = rg[64 + 64 * k: 128 + 64 * k].copy()
                    assert int(h[40:48].view("<u8")[0]) == r and int(h[48:56].view("<u8")[0]) == pb, (what, k)
                    want = exp[0].copy()
                    want[40:56] = h[40:56]
                    assert np.array_equal(h, want), (what, k)
                    assert np.array_equal(dcr.dcr_ready_wait(ready, k, 0), h)
                if mode == 1 or stage == 0 or n_slices != 3:
                    continue
                buf, canon = g.canon_alloc(co)
                flags = torch.zeros(max(len(got[1]) // 32, 1), dtype=torch.uint8, device="cuda")
                prev = 0
                for k, (r, pb) in enumerate(pre):
                    hk = rg[64 + 64 * k: 128 + 64 * k].copy()
                    ar = g.apply(canon, hk, sb, flags, first=prev, n=r - prev)
                    assert int(ar["n_applied"]) == r - prev and int(ar["n_invalid"]) == 0, (what, k)
                    prev = r
                for t in range(len(co)):
                    assert np.array_equal(canon[t].cpu().numpy(), np.ascontiguousarray(cn[t]).view(np.uint8).ravel()), \
                        (what, t)


def test_pipelined_encode_refusals(gh):
    """The watermark region must be pinned host memory of the right size and
    alignment; refused before any launch.  A stream that outgrows its payload
    buffer stops publishing with DCR_E_CAPACITY."""
    say("pipelined encode refusals")
    lay = pipe_layout("random", 3)
    g = gh.Gpu(lay)
    sb = dcr.StreamBuffers(g.plan, "cuda")
    args = (g.plan, g.olds, g.news, 0, 7, 8, sb.header, sb.dir, sb.payload, sb.result, g.ws)
    for bad in (torch.zeros(dcr.ready_region_bytes(4), dtype=torch.uint8, device="cuda"),   # device memory
                torch.zeros(dcr.ready_region_bytes(4), dtype=torch.uint8),                  # pageable
                torch.zeros(64, dtype=torch.uint8, pin_memory=True)):                       # too small
        with pytest.raises(dcr.DcrError):
            dcr.dcr_encode_pipelined(*args, 4, bad)
    with pytest.raises(dcr.DcrError):
        dcr.dcr_encode_pipelined(*args, 0, torch.zeros(128, dtype=torch.uint8, pin_memory=True))
    torch.cuda.synchronize()
    small = dcr.StreamBuffers(g.plan, "cuda", payload_bytes=4096)
    ready = torch.zeros(dcr.ready_region_bytes(3), dtype=torch.uint8, pin_memory=True)
    dcr.dcr_encode_pipelined(g.plan, g.olds, g.news, 0, 7, 8, small.header, small.dir, small.payload, small.result,
                             g.ws, 3, ready)
    torch.cuda.synchronize()
    rg = ready.numpy()
    assert int(rg[8:12].view("<i4")[0]) == dcr.DCR_E_CAPACITY
    assert int(small.result_host()["status"]) == dcr.DCR_E_CAPACITY
    n = int(rg[12:16].view("<u4")[0])
    with pytest.raises(dcr.DcrError) as e:
        dcr.dcr_ready_wait(ready, n - 1, 1000)
    assert e.value.code == dcr.DCR_E_CAPACITY


def test_capacity_overflow(gh, orc):
    """Too-small buffers: status DCR_E_CAPACITY with the required sizes."""
    say("capacity overflow")
    lay = synth.random_layout(3, rate=0.2)
    olds, news, co, cn = pins.canon_lists(lay)
    h, d, p = oracle_stream(orc, lay, olds, news)
    g = gh.Gpu(lay, olds, news)
    for dcap, pcap in ((len(d) - 32, len(p)), (len(d), len(p) - 16), (32, 16)):
        for stage in stage_sizes(g):
            sb = g.encode(0, dir_bytes=dcap, payload_bytes=pcap, stage=stage)
            r = sb.result_host()
            assert int(r["status"]) == dcr.DCR_E_CAPACITY
            assert int(r["n_records"]) * 32 == len(d) and int(r["payload_bytes"]) == len(p)


def test_header_checks(gh):
    """Wrong base version, plan fingerprint or stream kind are refused on the host."""
    say("header checks")
    lay = synth.random_layout(5, rate=0.2)
    g = gh.Gpu(lay)
    sb = g.encode(0)
    hdr, d, p = g.stream_host(sb)
    olds, news, co, cn = pins.canon_lists(lay)
    buf, canon = g.canon_alloc(co)
    flags = torch.zeros(max(len(d) // 32, 1), dtype=torch.uint8, device="cuda")
    with pytest.raises(dcr.DcrError) as e:
        g.apply(canon, hdr, sb, flags, base=6)
    assert e.value.code == dcr.DCR_E_VERSION
    bad = hdr.copy(); bad[32] ^= 1
    with pytest.raises(dcr.DcrError) as e:
        g.apply(canon, bad, sb, flags)
    assert e.value.code == dcr.DCR_E_FORMAT
    with pytest.raises(dcr.DcrError) as e:
        g.retry(canon, hdr, sb)            # a DELTA stream is not a RETRY stream
    assert e.value.code == dcr.DCR_E_FORMAT
    got = gh.host(canon)
    for t in range(lay.n_tensors):
        assert np.array_equal(got[t], co[t])   # nothing was touched


def test_corrupt_records_refused(gh):
    """A record whose bitmap popcount or fields are wrong is refused on the
    device and its chunk left untouched; the other records still apply."""
    say("corrupt records")
    lay = synth.config1_layout(512, 512)
    old, new, _lr, _pos = synth.config1_values(lay, lr=synth.CFG1_LR)
    g = gh.Gpu(lay, [old], [new])
    sb = g.encode(0)
    hdr, d, p = g.stream_host(sb)
    ents = fmt.dirents(d)
    assert len(ents) >= 4
    # flip one bitmap bit of record 1 and the K of record 2
    sb.payload[ents[1]["off"]] ^= 0x01
    dd = sb.dir.clone()
    dd[2 * 32 + 8] ^= 0x01
    sb.dir.copy_(dd)
    buf, canon = g.canon_alloc([old])
    flags = torch.zeros(len(ents), dtype=torch.uint8, device="cuda")
    r = g.apply(canon, hdr, sb, flags)
    assert int(r["n_invalid"]) == 2 and int(r["first_invalid"]) == 1
    assert int(r["n_applied"]) == len(ents) - 2
    w = canon[0].cpu().numpy().view(np.uint16)
    E = 32768
    for i, e in enumerate(ents):
        sl = slice(e["c"] * E, (e["c"] + 1) * E)
        exp = old[sl] if i in (1, 2) else new[sl]
        assert np.array_equal(w[sl], exp), i
    assert flags[1].item() == 0 and flags[2].item() == 0 and flags[0].item() == 1


@pytest.mark.parametrize("whole_lines", (False, True))
@pytest.mark.parametrize("groups", (1000, 1003))
def test_rmw_probe(gh, groups, whole_lines):
    """The read-modify-write probes that bench.py times as the apply's
    ceilings (16-byte groups alone, or every touched 128-byte line whole)
    XOR their fixed mask into exactly the flagged 16-byte groups (a ragged
    last word of bits and a ragged last line included), and a second run
    restores the buffer."""
    say("rmw probe:", groups, "groups, whole lines" if whole_lines else "groups alone")
    rng = np.random.default_rng(5)
    host = rng.integers(0, 256, size=16 * groups, dtype=np.uint8)
    flags = rng.random(groups) < 0.3
    nb = (groups + 15) // 16 * 16
    bits = np.packbits(np.concatenate([flags, np.ones(nb - groups, bool)]), bitorder="little")
    buf = torch.from_numpy(host.copy()).cuda()
    bdev = torch.from_numpy(bits).cuda()
    synth.rmw_probe_gpu(buf, bdev, whole_lines=whole_lines)
    torch.cuda.synchronize()
    mask = np.array([0x00010001, 0x00800080, 0x01000100, 0x80008000], dtype="<u4").view(np.uint8)
    exp = host.reshape(groups, 16).copy()
    exp[flags] ^= mask
    assert np.array_equal(buf.cpu().numpy().reshape(groups, 16), exp)
    synth.rmw_probe_gpu(buf, bdev, whole_lines=whole_lines)
    torch.cuda.synchronize()
    assert np.array_equal(buf.cpu().numpy(), host)


def _line_mode_layout(seed):
    """Identity tensors around the apply's line-mode cases: densities on both
    sides of its threshold, ragged last chunks and groups, 1-byte and 2-byte
    elements, overwrite routes, and block-scaled tensors whose scale blocks
    are (64 BF16 = one 128-byte line) and are not (8 BF16) whole lines, and
    one whose block (96 BF16) is not a power of two.  Block-scaled chunks
    hold an XOR and an overwrite record: dense XOR with sparse and with
    dense overwrite blocks (both records in line mode, each writing whole
    only the lines the other leaves alone), and a 1-byte chunk whose XOR
    record is too large for the small-record stage."""
    rng = np.random.default_rng(seed)
    b = synth._Builder("lines", seed)
    olds, news = [], []

    def add(numel, w, rate, route=synth.ROUTE_AFFINE_XOR, scale_block=0, scale_rate=0.3):
        dt = {1: np.uint8, 2: np.uint16, 4: np.uint32}[w]
        st = -1
        if route == synth.ROUTE_BLOCK_SCALED:
            ns = (numel + scale_block - 1) // scale_block
            st = b.tensor(f"s{len(olds)}", ns, 4, synth.ROUTE_OVERWRITE)
            s = b.shard(ns, 4)
            b.seg(st, s, 0, 0, [ns], [1], [1])
            so = rng.integers(0, 1 << 32, size=ns, dtype=np.uint64).astype(np.uint32)
            sn = so.copy()
            hit = rng.random(ns) < scale_rate
            sn[hit] ^= 1
            olds.append(so)
            news.append(sn)
        t = b.tensor(f"t{len(olds)}", numel, w, route, st, scale_block)
        s = b.shard(numel, w)
        b.seg(t, s, 0, 0, [numel], [1], [1])
        o = rng.integers(0, 1 << (8 * w), size=numel, dtype=np.uint64).astype(dt)
        n = o.copy()
        ch = rng.random(numel) < rate
        n[ch] ^= rng.integers(1, 1 << (8 * w), size=int(ch.sum()), dtype=np.uint64).astype(dt)
        olds.append(o)
        news.append(n)

    add(2 * 32768 + 1003, 2, 0.03)                       # ragged last chunk and group
    add(40000, 2, 0.013, synth.ROUTE_OVERWRITE)          # just above the threshold
    add(3 * 32768, 2, 0.011)                             # just below it
    add(65536 + 777, 1, 0.05)
    add(50000, 2, 0.05, synth.ROUTE_BLOCK_SCALED, 8)     # blocks of 16 bytes: group path
    add(50000, 2, 0.05, synth.ROUTE_BLOCK_SCALED, 64)    # blocks of one line: line path
    add(70000, 2, 0.05, synth.ROUTE_BLOCK_SCALED, 96)    # blocks of 12 groups (not a power of two)
    add(1000, 2, 0.2)
    add(3 * 32768, 2, 0.05, synth.ROUTE_BLOCK_SCALED, 64, 0.03)    # dense XOR, sparse overwrite blocks
    add(3 * 32768, 2, 0.1, synth.ROUTE_BLOCK_SCALED, 64, 0.3)      # both dense enough for line mode
    add(2 * 32768, 2, 0.3, synth.ROUTE_BLOCK_SCALED, 64, 0.02)     # XOR record past the small stage
    add(2 * 65536, 1, 0.2, synth.ROUTE_BLOCK_SCALED, 128, 0.05)    # 1-byte elements, both records
    lay = b.build()
    lay.values = (olds, news)
    return lay, olds, news


@pytest.mark.parametrize("align", [16, 256])
def test_apply_line_mode_edges(gh, orc, align):
    """Apply and retry give the new tensors bit for bit when the canonical
    tensors are packed at 16-byte offsets (no 128-byte aligned chunk: group
    path, neighbours sharing lines) and at 256-byte offsets (line path for
    the dense records); the streams equal the oracle's.  The index-list
    stream (sparse records as lists: no line mode beside them) applies to
    new too."""
    lay, olds, news = _line_mode_layout(11)
    say("line-mode edges, canonical alignment", align)
    g = gh.Gpu(lay, olds, news)
    for mode in (0, 1):
        sb = g.encode(mode)
        got = g.stream_host(sb)
        assert_same_stream(got, oracle_stream(orc, lay, olds, news, mode), f"mode {mode}")
    sb = g.encode(0)
    hdr, d, p = g.stream_host(sb)
    n = len(d) // 32
    buf, canon = g.canon_alloc(olds, align=align)
    flags = torch.zeros(max(n, 1), dtype=torch.uint8, device="cuda")
    r = g.apply(canon, hdr, sb, flags)
    assert int(r["n_applied"]) == n and int(r["n_invalid"]) == 0
    for v, e in zip(gh.host(canon), news):
        assert np.array_equal(v, e.view(np.uint8)), "apply"
    lsb = g.encode(dcr.ENC_INDEX_LISTS)
    lh, ld, _lp = g.stream_host(lsb)
    nl = len(ld) // 32
    buf, canon = g.canon_alloc(olds, align=align)
    lflags = torch.zeros(max(nl, 1), dtype=torch.uint8, device="cuda")
    r = g.apply(canon, lh, lsb, lflags)
    assert int(r["n_applied"]) == nl and int(r["n_invalid"]) == 0
    for v, e in zip(gh.host(canon), news):
        assert np.array_equal(v, e.view(np.uint8)), "apply, index lists"
    # kill at half the records from old, then the overwrite retry
    buf, canon = g.canon_alloc(olds, align=align)
    flags.zero_()
    g.apply(canon, hdr, sb, flags, 0, n // 2)
    rsb = g.encode(1)
    rh, _rd, _rp = g.stream_host(rsb)
    r = g.retry(canon, rh, rsb)
    assert int(r["n_invalid"]) == 0
    for v, e in zip(gh.host(canon), news):
        assert np.array_equal(v, e.view(np.uint8)), "retry"


@pytest.mark.parametrize("align", [16, 256])
def test_apply_pairs(gh, orc, align):
    """Chunks with an XOR and an overwrite record (block-scaled tensors): the
    XOR record's workgroup applies both (the overwrite record's groups, then
    its own, whole lines only where the overwrite record marks none).  Each
    case equals the oracle's apply from the same state and flags, byte for
    byte, with the same counts: every record fresh; the overwrite records of
    some pairs, the XOR records of others and both records of others already
    flagged (skipped); the XOR record of one pair, the overwrite record of
    another and both records of a third corrupted (refused, while the other
    record of the pair applies); and calls split between the two records of
    a pair.  Canonical tensors at 16-byte offsets (group path) and at
    256-byte offsets (line mode)."""
    lay, olds, news = _line_mode_layout(11)
    say("apply pairs, canonical alignment", align)
    g = gh.Gpu(lay, olds, news)
    sb = g.encode(0)
    hdr, d, p = g.stream_host(sb)
    ents = fmt.dirents(d)
    n = len(ents)
    pairs = [i for i in range(n - 1) if (ents[i]["t"], ents[i]["c"]) == (ents[i + 1]["t"], ents[i + 1]["c"])
             and ents[i]["w"] == 2]
    assert len(pairs) >= 10, len(pairs)
    co = [np.ascontiguousarray(x).view(np.uint8).reshape(-1).copy() for x in olds]

    def check(what, flags0, payload=None, calls=((0, None),), refused=(), dirb=None):
        # the oracle refuses a whole stream with a bad record: its expected
        # state skips the refused records instead (flagged beforehand)
        if payload is not None:
            sb.payload[:len(payload)].copy_(torch.from_numpy(payload))
        if dirb is not None:
            sb.dir[:len(dirb)].copy_(torch.from_numpy(dirb))
        buf, canon = g.canon_alloc(co, align=align)
        fl = torch.from_numpy(flags0.copy()).cuda()
        res = [g.apply(canon, hdr, sb, fl, f0, cnt) for f0, cnt in calls]
        W = [x.copy() for x in co]
        fo = flags0.copy()
        fo[list(refused)] = 1
        for f0, cnt in calls:
            assert orc.apply(lay.tensors, W, hdr, d, p, fo, f0, cnt, expected_base_version=7) == 0
        fo[list(refused)] = 0
        got = gh.host(canon)
        for t in range(lay.n_tensors):
            assert np.array_equal(got[t], W[t]), (what, t)
        assert np.array_equal(fl.cpu().numpy(), fo), what
        if payload is not None:
            sb.payload[:len(p)].copy_(torch.from_numpy(p))
        if dirb is not None:
            sb.dir[:len(d)].copy_(torch.from_numpy(d))
        return res

    zero = np.zeros(n, np.uint8)
    res = check("fresh", zero)
    assert int(res[0]["n_applied"]) == n and int(res[0]["n_invalid"]) == 0
    f = zero.copy()
    for i in pairs[0::3]:
        f[i + 1] = 1
    for i in pairs[1::3]:
        f[i] = 1
    for i in pairs[2::6]:
        f[i] = f[i + 1] = 1
    res = check("flagged", f)
    assert int(res[0]["n_skipped"]) == int(f.sum())
    assert int(res[0]["n_applied"]) == n - int(f.sum())
    bad = p.copy()
    bad[ents[pairs[0]]["off"]] ^= 0x01           # an XOR record's bitmap: popcount no longer K
    bad[ents[pairs[1] + 1]["off"]] ^= 0x01       # an overwrite record's bitmap
    bad[ents[pairs[2]]["off"]] ^= 0x01           # both records of a third pair
    bad[ents[pairs[2] + 1]["off"]] ^= 0x01
    refused = (pairs[0], pairs[1] + 1, pairs[2], pairs[2] + 1)
    res = check("corrupt", zero, payload=bad, refused=refused)
    assert int(res[0]["n_invalid"]) == 4 and int(res[0]["first_invalid"]) == pairs[0]
    assert int(res[0]["n_applied"]) == n - 4
    # a directory entry of a pair that fails its structural checks (K one
    # too many): not a fused pair, that record refused by its own workgroup
    # and the other record applied by its own
    bad_dir = d.copy()
    for i in (pairs[3] + 1, pairs[4]):
        k = bad_dir[32 * i + 8:32 * i + 12].view("<u4")
        k[0] += 1
    res = check("bad entries", zero, dirb=bad_dir, refused=(pairs[3] + 1, pairs[4]))
    assert int(res[0]["n_invalid"]) == 2 and int(res[0]["first_invalid"]) == pairs[3] + 1
    assert int(res[0]["n_applied"]) == n - 2
    i = pairs[len(pairs) // 2]
    check("split", zero, calls=((0, i + 1), (i + 1, n - i - 1)))


def test_graph_replay(gh, orc):
    """Encode (staged) and apply captured once in a HIP graph (torch's graph
    capture over the library's own launches) and replayed: every replay,
    with eager work between replays, gives the oracle's stream byte for byte
    and patches a fresh copy of the old tensors into the new ones.  The
    address tables are pinned PtrTables that outlive the graph (the copy of a
    table is a node of the graph and reads it at each replay)."""
    lay = synth.llama_layout(hidden=256, layers=2, ffn=640, n_q=8, n_kv=4, head_dim=32, vocab=1000, tp=4,
                             rate=0.03)
    say("graph replay: scaled TP=4 llama, 3 %")
    olds, news = lay.shards_host(0), lay.shards_host(1)
    g = gh.Gpu(lay, olds, news)
    exp = oracle_stream(orc, lay, olds, news, 0)
    n = len(exp[1]) // 32
    canon_new = lay.assemble([torch.from_numpy(x.view(np.int16)) for x in news])
    canon_old = lay.assemble([torch.from_numpy(x.view(np.int16)) for x in olds])
    buf, canon = g.canon_alloc()
    old_img = torch.cat([c.reshape(-1).view(torch.uint8) for c in canon_old]).cuda() if canon_old else None

    def reset_receiver():
        off = 0
        for v in canon:
            v.copy_(old_img[off:off + v.numel()])
            off += v.numel()

    ws = dcr.workspace(g.plan, "cuda", int(g.plan.info.max_payload_bytes))
    sb = dcr.StreamBuffers(g.plan, "cuda")
    ot, nt, ct = dcr.PtrTable(g.olds), dcr.PtrTable(g.news), dcr.PtrTable(canon)
    flags = torch.zeros(max(n, 1), dtype=torch.uint8, device="cuda")
    res = torch.zeros(32, dtype=torch.uint8, device="cuda")
    hdr = exp[0]
    # eager warm-up on the side stream torch captures on
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dcr.dcr_encode(g.plan, ot, nt, 0, 7, 8, sb.header, sb.dir, sb.payload, sb.result, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dcr.dcr_encode(g.plan, ot, nt, 0, 7, 8, sb.header, sb.dir, sb.payload, sb.result, ws)
        flags.zero_()
        dcr.dcr_apply(g.plan, ct, hdr, sb.dir, sb.payload, flags, 0, n, 7, res, g.ws)
    for rep in range(4):
        say("graph replay", rep)
        sb.dir.fill_(0xEE)
        sb.payload[: len(exp[2]) + 64].fill_(0xEE)
        reset_receiver()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = g.stream_host(sb)
        assert_same_stream(got, exp, f"replay {rep}")
        ar = dcr.apply_result(res)
        assert int(ar["n_applied"]) == n and int(ar["n_invalid"]) == 0, (rep, ar)
        for v, e in zip(canon, canon_new):
            assert torch.equal(v.view(torch.int16).cpu(), e.reshape(-1)), f"replay {rep}: apply"
        # eager work between replays: a RETRY encode into other buffers
        other = g.encode(1)
        assert int(other.result_host()["status"]) == 0
    del graph


def test_compact_staging(gh, orc):
    """A staging area smaller than every chunk's slot but at least
    compact_stage_bytes is used compactly (each chunk claims its records'
    bytes in one of 64 partitions; a chunk that finds no room is encoded
    again at its place after the fix-up).  On config 1's tensor (512 chunks)
    with the smallest such area, one 16 bytes larger, one twice the stream's
    payload and one just short of the full worst case, the DELTA and RETRY
    streams equal the oracle's byte for byte; from twice the payload up no
    chunk is encoded twice, and with a full area none ever is."""
    lay = synth.config1_layout()
    old, new, _lr, _pos = synth.config1_values(lay, lr=synth.CFG1_LR)
    g = gh.Gpu(lay, [old], [new])
    info = g.plan.info
    win, full = int(info.compact_stage_bytes), int(info.max_payload_bytes)
    assert 0 < win < full
    for mode in (0, 1):
        exp = oracle_stream(orc, lay, [old], [new], mode)
        pb = len(exp[2])
        for stage in (win, win + 16, 2 * pb, full - 16, full):
            sb = g.encode(mode, stage=stage)
            assert_same_stream(g.stream_host(sb), exp, f"mode {mode} stage {stage}")
            re = int(sb.result_host()["n_reencoded"])
            say("compact staging", mode, stage, pb, re)
            if stage >= 2 * pb:
                assert re == 0, (mode, stage)
    # the index-list layout and the partial retry stage the same way
    rc, lh, ld, lp = orc.encode(lay.tensors, lay.segments, [old], [new], mode=dcr.ENC_INDEX_LISTS,
                                base_version=7, new_version=8)
    assert rc == 0
    assert_same_stream(g.stream_host(g.encode(dcr.ENC_INDEX_LISTS, stage=win)), (lh, ld, lp), "lists, compact")
    sb = g.encode(0)
    hdr, d, _p = g.stream_host(sb)
    n = len(d) // 32
    buf, canon = g.canon_alloc([old])
    flags = torch.zeros(n, dtype=torch.uint8, device="cuda")
    g.apply(canon, hdr, sb, flags, 0, n // 3)
    rc, eh, ed, ep = orc.encode_retry_partial(lay.tensors, lay.segments, [old], [new], hdr, d, flags.cpu().numpy(),
                                               base_version=7, new_version=8)
    assert rc == 0
    assert_same_stream(g.stream_host(g.encode_retry_partial(hdr, sb, flags, stage=win)), (eh, ed, ep),
                       "partial retry, compact")


@pytest.mark.parametrize("frac", [1.0, 0.6, 0.3])
def test_compact_staging_overflow(gh, orc, frac):
    """Compact staging with too little room: config 1's tensor (512 chunks)
    with a fraction `frac` of its elements changed in random bits (records
    near their worst case at 1.0) and the smallest compact area, so that
    chunks find their partition full and are encoded again after the
    fix-up.  DELTA, RETRY and index-list streams equal the oracle's byte for
    byte, and the count of chunks encoded again is nonzero whenever the
    stream's payload exceeds the area."""
    lay = synth.config1_layout()
    old, _new, _lr, _pos = synth.config1_values(lay, lr=synth.CFG1_LR)
    rng = np.random.default_rng(int(frac * 1000) + 17)
    x = rng.integers(1, 1 << 16, old.size, dtype=np.uint16)
    x[rng.random(old.size) >= frac] = 0
    new = old ^ x
    g = gh.Gpu(lay, [old], [new])
    win = int(g.plan.info.compact_stage_bytes)
    for mode in (0, 1, dcr.ENC_INDEX_LISTS):
        exp = oracle_stream(orc, lay, [old], [new], mode)
        sb = g.encode(mode, stage=win)
        r = sb.result_host()
        say("compact overflow", frac, mode, int(r["payload_bytes"]), win, int(r["n_reencoded"]))
        assert_same_stream(g.stream_host(sb), exp, f"frac {frac} mode {mode}")
        if int(r["payload_bytes"]) > win:
            assert int(r["n_reencoded"]) > 0
        assert int(r["n_reencoded"]) <= 512
