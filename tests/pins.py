"""Pins of the CPU oracle: checks against what the pages and the mathematics fix.

Each ``pin_*`` takes an ``Oracle`` and raises AssertionError on a mismatch.
They are run against the real oracle (test_oracle_pins.py) and against copies
of the oracle with planted mistakes (test_oracle_mutants.py), each of which
must fail at least one pin.

Sources of the facts pinned:
  * new = old XOR (old XOR new) on a flat bit buffer, no arithmetic involved:
    humansand "weight teleportation" page, "Delta update algebra".
  * changes are detected on stored bits, so +0 -> -0 is a change that float
    equality misses: tokendh blog, "shard owner" section and closing notes.
  * a XOR applied twice undoes itself, hence unique ids / dedup: tokendh blog,
    "XOR or overwrite" section.
  * overwrite is idempotent, so a whole-set overwrite retry heals a partial
    apply: tokendh blog, "no backup copy" section; ai.info abstract.
  * XOR masks are smaller than overwrites: ai-feeds summary, "key modules" 3.
  * changes are projected to canonical coordinates by a fixed affine map:
    ai-feeds summary, "key modules" 1.
"""
import os

import numpy as np

from bit_exact_xor_amd import synth
from oracle.oracle import E_FORMAT as O_E_FORMAT
from tests import fmt

MODE_DELTA, MODE_RETRY = 0, 1

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------- helpers

def canon_lists(lay):
    """Canonical old / new per tensor as uint8 arrays, built by library ops."""
    olds, news = lay.shards_host(0), lay.shards_host(1)
    co = [np.ascontiguousarray(np.asarray(x)).view(np.uint8).reshape(-1).copy() for x in lay.assemble(olds)]
    cn = [np.ascontiguousarray(np.asarray(x)).view(np.uint8).reshape(-1).copy() for x in lay.assemble(news)]
    return olds, news, co, cn


def words_of(buf, w):
    return np.ascontiguousarray(buf).view({1: np.uint8, 2: np.uint16, 4: np.uint32}[w]).astype(np.uint32)


def expected_changes(lay, co, cn, mode=0):
    """Definition: changed iff stored bits differ; kind by route; word XOR/new."""
    out = []
    T = lay.tensors
    for t in range(len(T)):
        w, route = int(T[t]["elem_bytes"]), int(T[t]["route"])
        o, n = words_of(co[t], w), words_of(cn[t], w)
        ch = np.nonzero(o != n)[0]
        if mode == 1:
            kind = np.ones(len(ch), dtype=int)
        elif route == 0:
            kind = np.zeros(len(ch), dtype=int)
        elif route == 1:
            kind = np.ones(len(ch), dtype=int)
        else:
            st, sb = int(T[t]["scale_tensor"]), int(T[t]["scale_block"])
            so, sn = words_of(co[st], 4), words_of(cn[st], 4)
            kind = (so[ch // sb] != sn[ch // sb]).astype(int)
        word = np.where(kind == 0, o[ch] ^ n[ch], n[ch])
        E = 65536 // w
        for k in (0, 1):
            sel = kind == k
            for c in np.unique(ch[sel] // E):
                m = sel & (ch // E == c)
                out.append((t, int(c), k, ch[m], word[m]))
    out.sort(key=lambda r: (r[0], r[1], r[2]))
    return out


def check_stream_against_definition(lay, co, cn, hdr, d, p, mode=0):
    T = lay.tensors
    numels = [int(x) for x in T["numel"]]
    widths = [int(x) for x in T["elem_bytes"]]
    got = fmt.decode_stream(hdr, d, p, numels, widths)
    exp = expected_changes(lay, co, cn, mode)
    assert len(got) == len(exp), (len(got), len(exp))
    for g, e in zip(got, exp):
        assert g[:3] == e[:3], (g[:3], e[:3])
        assert np.array_equal(g[3], e[3])
        assert np.array_equal(g[4].astype(np.uint32), e[4].astype(np.uint32))
    h = fmt.header(hdr)
    assert h["magic"] == fmt.MAGIC and h["n_records"] == len(exp) and h["kind"] == mode
    assert h["payload_bytes"] == len(p)


def encode_ok(orc, lay, olds, news, mode=0, base=7, new=8):
    rc, hdr, d, p = orc.encode(lay.tensors, lay.segments, olds, news, mode=mode,
                               base_version=base, new_version=new)
    assert rc == 0, rc
    return hdr, d, p


# ------------------------------------------------------------------- pins

def pin_roundtrip_random(orc, seeds=range(12)):
    """apply(old, encode(old, new)) == new, and the stream decodes to exactly
    {(i, old^new or new)} by the definition, on random layouts."""
    for seed in seeds:
        lay = synth.random_layout(seed)
        olds, news, co, cn = canon_lists(lay)
        hdr, d, p = encode_ok(orc, lay, olds, news)
        check_stream_against_definition(lay, co, cn, hdr, d, p)
        W = [x.copy() for x in co]
        flags = np.zeros(max(len(d) // 32, 1), np.uint8)
        assert orc.apply(lay.tensors, W, hdr, d, p, flags, expected_base_version=7) == 0
        for t in range(lay.n_tensors):
            assert np.array_equal(W[t], cn[t]), (seed, t)


def pin_width_sets(orc):
    """Layouts of every set of element widths, 4-byte overwrite tensors also
    on their own and split or transposed: both streams decode to the
    definition, apply gives new and the overwrite retry gives new."""
    for ws in range(1, 8):
        lay = synth.width_set_layout(ws)
        olds, news, co, cn = canon_lists(lay)
        for mode in (MODE_DELTA, MODE_RETRY):
            hdr, d, p = encode_ok(orc, lay, olds, news, mode=mode)
            check_stream_against_definition(lay, co, cn, hdr, d, p, mode)
            W = [x.copy() for x in co]
            if mode == MODE_DELTA:
                flags = np.zeros(max(len(d) // 32, 1), np.uint8)
                assert orc.apply(lay.tensors, W, hdr, d, p, flags, expected_base_version=7) == 0
            else:
                assert orc.retry(lay.tensors, W, hdr, d, p, expected_base_version=7) == 0
            for t in range(lay.n_tensors):
                assert np.array_equal(W[t], cn[t]), (ws, mode, t)


def pin_xor_involution(orc, seeds=range(4)):
    """Applying a XOR-only stream twice (flags reset) restores old; with the
    flags kept, the second apply is a no-op (dedup)."""
    for seed in seeds:
        lay = synth.random_layout(100 + seed, allow_block_scaled=False)
        lay.tensors["route"][:] = 0
        olds, news, co, cn = canon_lists(lay)
        hdr, d, p = encode_ok(orc, lay, olds, news)
        n = len(d) // 32
        W = [x.copy() for x in co]
        flags = np.zeros(max(n, 1), np.uint8)
        assert orc.apply(lay.tensors, W, hdr, d, p, flags, expected_base_version=7) == 0
        assert orc.apply(lay.tensors, W, hdr, d, p, flags, expected_base_version=7) == 0
        for t in range(lay.n_tensors):
            assert np.array_equal(W[t], cn[t])           # duplicate skipped
        flags[:] = 0
        assert orc.apply(lay.tensors, W, hdr, d, p, flags, expected_base_version=7) == 0
        for t in range(lay.n_tensors):
            assert np.array_equal(W[t], co[t])           # XOR twice == old


def pin_retry_idempotent(orc, seeds=range(4)):
    """From any prior state (untouched, half applied, a torn record, XOR
    records applied twice) the overwrite retry gives new, and retrying twice
    equals retrying once."""
    for seed in seeds:
        lay = synth.random_layout(200 + seed)
        olds, news, co, cn = canon_lists(lay)
        hdr, d, p = encode_ok(orc, lay, olds, news)
        rh, rd, rp = encode_ok(orc, lay, olds, news, mode=1)
        check_stream_against_definition(lay, co, cn, rh, rd, rp, mode=1)
        n = len(d) // 32
        states = []
        states.append([x.copy() for x in co])                       # untouched
        W = [x.copy() for x in co]
        f = np.zeros(max(n, 1), np.uint8)
        orc.apply(lay.tensors, W, hdr, d, p, f, 0, n // 2, expected_base_version=7)
        states.append(W)                                            # killed at 50 %
        if n:
            W = [x.copy() for x in co]
            ents = fmt.dirents(d)
            r = n // 2
            orc.apply_record_part(lay.tensors, W, d, p, r, 0, max(ents[r]["K"] // 2, 1))
            states.append(W)                                        # torn record
            W = [x.copy() for x in co]
            f = np.zeros(n, np.uint8)
            orc.apply(lay.tensors, W, hdr, d, p, f, 0, n, expected_base_version=7)
            f[::2] = 0
            orc.apply(lay.tensors, W, hdr, d, p, f, 0, n, expected_base_version=7)
            states.append(W)                                        # duplicated XORs
        for W in states:
            assert orc.retry(lay.tensors, W, rh, rd, rp, expected_base_version=7) == 0
            once = [x.copy() for x in W]
            assert orc.retry(lay.tensors, W, rh, rd, rp, expected_base_version=7) == 0
            for t in range(lay.n_tensors):
                assert np.array_equal(W[t], cn[t])
                assert np.array_equal(W[t], once[t])


def pin_retry_partial(orc, seeds=range(3)):
    """Partial retry (only chunks with an unflagged DELTA record are sent
    again): all flags clear gives the full RETRY stream byte for byte, all
    set gives an empty one; after a kill at record k (optionally with record k
    torn) the stream holds exactly the chunks of records k.. (read from the
    DELTA directory), each with the full RETRY stream's record, and applying
    it heals the receiver to new."""
    for seed in seeds:
        lay = synth.random_layout(900 + seed)
        olds, news, co, cn = canon_lists(lay)
        hdr, d, p = encode_ok(orc, lay, olds, news)
        rh, rd, rp = encode_ok(orc, lay, olds, news, mode=1)
        n = len(d) // 32
        ents = fmt.dirents(d)
        full = {(e["t"], e["c"]): rp[e["off"]:e["off"] + e["size"]] for e in fmt.dirents(rd)}

        def partial(flags):
            rc, h2, d2, p2 = orc.encode_retry_partial(lay.tensors, lay.segments, olds, news, hdr, d, flags,
                                                       base_version=7, new_version=8)
            assert rc == 0
            return h2, d2, p2

        h0, d0, p0 = partial(np.zeros(max(n, 1), np.uint8))
        assert np.array_equal(h0, rh) and np.array_equal(d0, rd) and np.array_equal(p0, rp)
        h1, d1, p1 = partial(np.ones(max(n, 1), np.uint8))
        assert len(d1) == 0 and len(p1) == 0 and int(h1[40:48].view("<u8")[0]) == 0
        for k in sorted({0, n // 3, n // 2, max(n - 1, 0)}):
            for torn in (False, True):
                if torn and k >= n:
                    continue
                W = [x.copy() for x in co]
                f = np.zeros(max(n, 1), np.uint8)
                orc.apply(lay.tensors, W, hdr, d, p, f, 0, k, expected_base_version=7)
                if torn:
                    orc.apply_record_part(lay.tensors, W, d, p, k, 0, max(ents[k]["K"] // 2, 1))
                hp, dp, pp = partial(f)
                got = fmt.dirents(dp)
                want = sorted({(e["t"], e["c"]) for r, e in enumerate(ents) if r >= k})
                assert [(e["t"], e["c"]) for e in got] == want, (seed, k)
                for e in got:
                    assert np.array_equal(pp[e["off"]:e["off"] + e["size"]], full[(e["t"], e["c"])])
                assert len(pp) <= len(rp)
                assert orc.retry(lay.tensors, W, hp, dp, pp, expected_base_version=7) == 0
                for t in range(lay.n_tensors):
                    assert np.array_equal(W[t], cn[t]), (seed, k, torn, t)
        # a RETRY header, or an entry naming no chunk, is refused
        rc, *_ = orc.encode_retry_partial(lay.tensors, lay.segments, olds, news, rh, d, np.zeros(max(n, 1), np.uint8))
        assert rc == O_E_FORMAT
        if n:
            bad = d.copy()
            bad[0:4] = np.frombuffer(np.uint32(lay.n_tensors).tobytes(), np.uint8)
            rc, *_ = orc.encode_retry_partial(lay.tensors, lay.segments, olds, news, hdr, bad, np.zeros(n, np.uint8))
            assert rc == O_E_FORMAT


def pin_index_lists(orc, seeds=range(6)):
    """Index-list layout (encode option): the same records as the bitmap
    stream in the same order, each in list layout exactly when 2K bytes
    (padded) are fewer than the padded bitmap; a list record is the bitmap
    record with the bitmap replaced by the ascending indices of its set bits
    (everything after it byte-identical); offsets stay contiguous; apply,
    XOR involution and retry work on it; malformed lists are refused."""
    for seed in seeds:
        lay = synth.random_layout(1200 + seed, rate=[0.002, 0.03, 0.2][seed % 3])
        olds, news, co, cn = canon_lists(lay)
        numels = [int(t["numel"]) for t in lay.tensors]
        widths = [int(t["elem_bytes"]) for t in lay.tensors]
        for mode in (MODE_DELTA, MODE_RETRY):
            bh, bd, bp = encode_ok(orc, lay, olds, news, mode=mode)
            rc, lh, ld, lp = orc.encode(lay.tensors, lay.segments, olds, news, mode=mode | 0x100,
                                        base_version=7, new_version=8)
            assert rc == 0
            assert np.array_equal(lh[:40], bh[:40]) and int(lh[40:48].view("<u8")[0]) == len(bd) // 32
            be, le = fmt.dirents(bd), fmt.dirents(ld)
            assert len(be) == len(le)
            off = 0
            for b, l in zip(be, le):
                for key in ("t", "c", "K", "kind", "hi_mode", "w", "H"):
                    assert b[key] == l[key], (seed, key)
                E = 65536 // b["w"]
                n_c = min(E, numels[b["t"]] - b["c"] * E)
                nb = (n_c + 7) // 8
                want_list = (2 * b["K"] + 15) // 16 * 16 < (nb + 15) // 16 * 16
                assert l["layout"] == (1 if want_list else 0), (seed, b["K"], n_c)
                assert l["off"] == off
                off += l["size"]
                rb = bp[b["off"]:b["off"] + b["size"]]
                rl = lp[l["off"]:l["off"] + l["size"]]
                if not want_list:
                    assert np.array_equal(rb, rl)
                    continue
                head_b, head_l = (nb + 15) // 16 * 16, (2 * b["K"] + 15) // 16 * 16
                assert l["size"] == b["size"] - head_b + head_l
                bits = np.unpackbits(rb[:nb], bitorder="little")[:n_c]
                idx = np.nonzero(bits)[0].astype("<u2")
                assert np.array_equal(rl[:2 * b["K"]], idx.view(np.uint8))
                assert not rl[2 * b["K"]:head_l].any()
                assert np.array_equal(rl[head_l:], rb[head_b:])
            assert off == len(lp)
            assert fmt.decode_stream(lh, ld, lp, numels, widths).__len__() == len(be)
            if mode == MODE_DELTA:
                W = [x.copy() for x in co]
                f = np.zeros(max(len(le), 1), np.uint8)
                assert orc.apply(lay.tensors, W, lh, ld, lp, f, expected_base_version=7) == 0
                for t in range(lay.n_tensors):
                    assert np.array_equal(W[t], cn[t])
                if all(e["kind"] == 0 for e in le):
                    f[:] = 0
                    assert orc.apply(lay.tensors, W, lh, ld, lp, f, expected_base_version=7) == 0
                    for t in range(lay.n_tensors):
                        assert np.array_equal(W[t], co[t])
            else:
                W = [x.copy() for x in co]
                assert orc.retry(lay.tensors, W, lh, ld, lp, expected_base_version=7) == 0
                for t in range(lay.n_tensors):
                    assert np.array_equal(W[t], cn[t])
            lists = [i for i, e in enumerate(le) if e["layout"] == 1 and e["K"] >= 2]
            if lists:
                e = le[lists[0]]
                bad = lp.copy()       # two indices swapped: not ascending
                a0 = e["off"]
                bad[a0:a0 + 2], bad[a0 + 2:a0 + 4] = lp[a0 + 2:a0 + 4].copy(), lp[a0:a0 + 2].copy()
                assert orc.validate(lay.tensors, lh, ld, bad, 7) == O_E_FORMAT
                bad = ld.copy()       # unknown layout
                bad[lists[0] * 32 + 15] = 2
                assert orc.validate(lay.tensors, lh, bad, lp, 7) == O_E_FORMAT


def pin_signed_zero(orc):
    """64 forced +0 <-> -0 flips are all encoded with mask 0x8000, and float
    equality on BF16 misses exactly those 64."""
    import torch
    lay = synth.config1_layout(512, 512)
    old, new, _lr, pos = synth.config1_values(lay, lr=synth.CFG1_LR)
    hdr, d, p = encode_ok(orc, lay, [old], [new])
    recs = fmt.decode_stream(hdr, d, p, [old.size], [2])
    got = {}
    for (_t, _c, _k, idx, words) in recs:
        got.update(zip(idx.tolist(), words.tolist()))
    for q in pos.tolist():
        assert got.get(q) == 0x8000, q
    to = torch.from_numpy(old.view(np.int16)).view(torch.bfloat16)
    tn = torch.from_numpy(new.view(np.int16)).view(torch.bfloat16)
    float_eq_changed = set(torch.nonzero(to != tn).reshape(-1).tolist())
    bit_changed = set(np.nonzero(old != new)[0].tolist())
    missed = bit_changed - float_eq_changed
    assert missed == set(pos.tolist()), (len(missed), len(pos))
    assert bit_changed == set(got.keys())


def pin_xor_not_larger(orc, seeds=range(6)):
    """Per chunk, a XOR record's payload is never larger than the overwrite
    record for the same change set."""
    for seed in seeds:
        lay = synth.random_layout(300 + seed, allow_block_scaled=False)
        lay.tensors["route"][:] = 0
        olds, news, co, cn = canon_lists(lay)
        _h, d, _p = encode_ok(orc, lay, olds, news)
        _rh, rd, _rp = encode_ok(orc, lay, olds, news, mode=1)
        x = {(e["t"], e["c"]): e for e in fmt.dirents(d)}
        o = {(e["t"], e["c"]): e for e in fmt.dirents(rd)}
        assert x.keys() == o.keys()
        for k in x:
            assert x[k]["K"] == o[k]["K"]
            assert x[k]["size"] <= o[k]["size"], (k, x[k], o[k])


def _one_tensor(n, w, route=0):
    T = np.zeros(1, dtype=synth.TENSOR_DT)
    T[0] = (n, w, route, -1, 0)
    S = np.zeros(1, dtype=synth.SEGMENT_DT)
    S[0]["ndim"] = 1
    S[0]["extent"] = [n, 1, 1, 1]
    S[0]["shard_stride"] = [1, 0, 0, 0]
    S[0]["canon_stride"] = [1, 0, 0, 0]
    return T, S


def _decode_one(orc, T, S, old, new, n, w):
    rc, hdr, d, p = orc.encode(T, S, [old], [new])
    assert rc == 0
    recs = fmt.decode_stream(hdr, d, p, [n], [w])
    idx = np.concatenate([r[3] for r in recs]) if recs else np.zeros(0, np.int64)
    words = np.concatenate([r[4] for r in recs]) if recs else np.zeros(0, np.uint32)
    return idx, words, (hdr, d, p)


def pin_bruteforce_subsets(orc):
    """n <= 12 elements: every subset of changed positions, random bits."""
    rng = np.random.default_rng(5)
    for n in (1, 2, 3, 7, 12):
        T, S = _one_tensor(n, 2)
        old = rng.integers(0, 1 << 16, size=n, dtype=np.uint64).astype(np.uint16)
        for sub in range(1 << n):
            sel = np.array([(sub >> i) & 1 for i in range(n)], dtype=bool)
            mask = rng.integers(1, 1 << 16, size=n, dtype=np.uint64).astype(np.uint16)
            new = np.where(sel, old ^ mask, old).astype(np.uint16)
            idx, words, _ = _decode_one(orc, T, S, old, new, n, 2)
            assert np.array_equal(idx, np.nonzero(sel)[0]), (n, sub)
            assert np.array_equal(words, (old ^ new)[sel].astype(np.uint32)), (n, sub)


def pin_u8_all_pairs(orc):
    """Every (old, new) pair of one byte: element j carries old=j>>8, new=j&255."""
    j = np.arange(65536)
    old, new = (j >> 8).astype(np.uint8), (j & 255).astype(np.uint8)
    for route in (0, 1):
        T, S = _one_tensor(65536, 1, route)
        idx, words, _ = _decode_one(orc, T, S, old, new, 65536, 1)
        sel = old != new
        assert np.array_equal(idx, np.nonzero(sel)[0])
        exp = (old ^ new) if route == 0 else new
        assert np.array_equal(words, exp[sel].astype(np.uint32))


def pin_bf16_special_olds(orc):
    """One BF16 old value against all 65536 new bit patterns, for signed
    zeros, smallest subnormals, +-1, +-max, +-Inf and a NaN."""
    olds = [0x0000, 0x8000, 0x0001, 0x8001, 0x3F80, 0xBF80, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80, 0x7FC1]
    new = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    T, S = _one_tensor(65536, 2)
    for o in olds:
        old = np.full(65536, o, dtype=np.uint16)
        idx, words, (hdr, d, p) = _decode_one(orc, T, S, old, new, 65536, 2)
        sel = old != new
        assert np.array_equal(idx, np.nonzero(sel)[0])
        assert np.array_equal(words, (old ^ new)[sel].astype(np.uint32))
        W = [old.view(np.uint8).copy()]
        f = np.zeros(len(d) // 32, np.uint8)
        assert orc.apply(T, W, hdr, d, p, f, expected_base_version=0) == 0
        assert np.array_equal(W[0].view(np.uint16), new)


def pin_partial_chunks(orc):
    """Tensors of 1..100 elements (one partial chunk), both widths and kinds."""
    rng = np.random.default_rng(9)
    for n in range(1, 101):
        for w in (1, 2):
            for route in (0, 1):
                T, S = _one_tensor(n, w, route)
                dt = np.uint8 if w == 1 else np.uint16
                old = rng.integers(0, 1 << (8 * w), size=n, dtype=np.uint64).astype(dt)
                new = np.where(rng.random(n) < 0.4, rng.integers(0, 1 << (8 * w), size=n,
                                                                 dtype=np.uint64).astype(dt), old)
                idx, words, (hdr, d, p) = _decode_one(orc, T, S, old, new, n, w)
                sel = old != new
                assert np.array_equal(idx, np.nonzero(sel)[0])
                exp = (old ^ new) if route == 0 else new
                assert np.array_equal(words, exp[sel].astype(np.uint32))
                for e in fmt.dirents(d):
                    assert e["size"] % 16 == 0 and e["off"] % 16 == 0


def pin_projection(orc):
    """Canonical tensors gathered through the affine segments equal those
    assembled from the shards with library cat / narrow / reshape, on a
    scaled-down TP=4 Llama layout and on random layouts."""
    lay = synth.llama_layout(hidden=256, layers=2, ffn=640, n_q=8, n_kv=4, head_dim=32,
                             vocab=1000, tp=4)
    import torch
    olds = lay.shards_host(0)
    ref = lay.assemble([torch.from_numpy(x.view(np.int16)) for x in olds])
    for t in range(lay.n_tensors):
        g = orc.gather(lay.tensors, lay.segments, olds, t)
        assert np.array_equal(g, ref[t].numpy().view(np.uint8)), lay.tensor_names[t]
    for seed in range(8):
        lay = synth.random_layout(400 + seed)
        olds = lay.shards_host(0)
        ref = lay.assemble(olds)
        for t in range(lay.n_tensors):
            g = orc.gather(lay.tensors, lay.segments, olds, t)
            assert np.array_equal(g, np.ascontiguousarray(ref[t]).view(np.uint8).reshape(-1))


def pin_coverage(orc):
    """Gaps and overlaps in the canonical coverage are rejected."""
    from oracle import oracle as O
    T, S = _one_tensor(100, 2)
    old = np.zeros(200, np.uint16)
    S2 = np.concatenate([S, S])
    S2[0]["extent"][0], S2[1]["extent"][0] = 60, 60
    S2[1]["shard_off"], S2[1]["canon_off"] = 60, 60          # gap? no: 60+60 > 100
    assert orc.encode(T, S2, [old], [old])[0] == O.E_INVAL    # out of range
    S2[1]["extent"][0] = 40
    assert orc.encode(T, S2, [old], [old])[0] == 0            # exact cover
    S2[1]["canon_off"] = 59                                   # overlap at 59, gap at 99
    assert orc.encode(T, S2, [old], [old])[0] == O.E_COVERAGE
    S2[1]["canon_off"], S2[1]["extent"][0] = 60, 39           # gap at 99
    assert orc.encode(T, S2, [old], [old])[0] == O.E_COVERAGE
    S2[1]["extent"][0], S2[1]["shard_off"] = 40, 170          # shard overrun
    assert orc.encode(T, S2, [old], [old])[0] == O.E_INVAL


def pin_counts(orc, seeds=range(6)):
    """Sum of K = popcount of all bitmaps = number of elements whose stored
    bits differ; record count and payload bytes equal their closed forms."""
    import torch
    for seed in seeds:
        lay = synth.random_layout(500 + seed)
        olds, news, co, cn = canon_lists(lay)
        hdr, d, p = encode_ok(orc, lay, olds, news)
        ents = fmt.dirents(d)
        total_changed = 0
        n_chunks_changed = 0
        closed = 0
        for t in range(lay.n_tensors):
            w = int(lay.tensors[t]["elem_bytes"])
            if co[t].size == 0:
                continue
            tt = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[w]
            a = torch.from_numpy(co[t].copy()).view(tt)
            b = torch.from_numpy(cn[t].copy()).view(tt)
            total_changed += int((a != b).sum())
        assert sum(e["K"] for e in ents) == total_changed
        pop = 0
        for e in ents:
            E = 65536 // e["w"]
            n_c = min(E, int(lay.tensors[e["t"]]["numel"]) - e["c"] * E)
            nb = (n_c + 7) // 8
            pop += int(np.unpackbits(p[e["off"]:e["off"] + nb]).sum())
        assert pop == total_changed
        # closed forms for an all-XOR or all-OW stream
        for e in ents:
            E = 65536 // e["w"]
            n_c = min(E, int(lay.tensors[e["t"]]["numel"]) - e["c"] * E)
            K, H, w = e["K"], e["H"], e["w"]
            sz = fmt.pad16((n_c + 7) // 8) + fmt.pad16(K)
            if w == 2 and e["kind"] == 0:
                sz += {0: 0, 1: fmt.pad16((K + 7) // 8) + fmt.pad16(H), 2: fmt.pad16(K)}[e["hi_mode"]]
            elif w == 2:
                sz += fmt.pad16(K)
            elif w == 4:
                sz += 3 * fmt.pad16(K)
            closed += sz
        assert closed == len(p) == fmt.header(hdr)["payload_bytes"]
        keys = {(e["t"], e["c"], e["kind"]) for e in ents}
        assert len(keys) == len(ents)
        n_chunks_changed = len(expected_changes(lay, co, cn))
        assert n_chunks_changed == len(ents)


def pin_hi_mode_rule(orc):
    """The high-byte mode is NONE without nonzero high bytes, else SPARSE iff
    presence bitmap + nonzero high bytes is strictly smaller than all K high
    bytes (16-byte padded sizes), else DENSE."""
    rng = np.random.default_rng(11)
    n = 32768
    T, S = _one_tensor(n, 2)
    old = rng.integers(0, 1 << 16, size=n, dtype=np.uint64).astype(np.uint16)
    for K, h in [(1, 0), (1, 1), (16, 1), (32, 1), (48, 16), (48, 17), (100, 1), (128, 2),
                 (128, 8), (1000, 60),
                 (1000, 600), (4096, 255), (4096, 256), (32768, 3000), (32768, 30000)]:
        pos = np.sort(rng.choice(n, K, replace=False))
        hip = rng.choice(K, h, replace=False)
        mask = np.zeros(n, np.uint16)
        mask[pos] = rng.integers(1, 256, size=K).astype(np.uint16)
        mask[pos[hip]] |= (rng.integers(1, 256, size=h).astype(np.uint16) << 8)
        new = old ^ mask
        _i, _w, (hdr, d, p) = _decode_one(orc, T, S, old, new, n, 2)
        e = fmt.dirents(d)[0]
        sparse = fmt.pad16((K + 7) // 8) + fmt.pad16(h)
        exp = 0 if h == 0 else (1 if sparse < fmt.pad16(K) else 2)
        assert e["hi_mode"] == exp, (K, h, e)
        assert e["H"] == {0: 0, 1: h, 2: K}[exp]


def pin_fingerprint(orc):
    """Plan fingerprint = FNV-1a-64 of the serialised tensor table (FNV
    reference vectors: empty -> cbf29ce484222325, 'a' -> af63dc4c8601ec8c)."""
    assert fmt.fnv1a64(b"") == 0xCBF29CE484222325
    assert fmt.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert fmt.fnv1a64(b"foobar") == 0x85944171F73967E8
    lay = synth.random_layout(7)
    T = np.zeros(len(lay.tensors), dtype=synth.TENSOR_DT)
    T[:] = lay.tensors
    assert orc.fingerprint(lay.tensors) == fmt.fnv1a64(T.tobytes())


def pin_validation(orc):
    """Corrupt streams are refused; a wrong base version is refused."""
    from oracle import oracle as O
    lay = synth.random_layout(3, rate=0.2)
    olds, news, co, cn = canon_lists(lay)
    hdr, d, p = encode_ok(orc, lay, olds, news)
    assert len(d) >= 64
    assert orc.validate(lay.tensors, hdr, d, p, 7) == 0
    assert orc.validate(lay.tensors, hdr, d, p, 6) == O.E_VERSION
    bad = hdr.copy(); bad[0] ^= 1
    assert orc.validate(lay.tensors, bad, d, p, 7) == O.E_FORMAT
    bad = hdr.copy(); bad[32] ^= 1
    assert orc.validate(lay.tensors, bad, d, p, 7) == O.E_FORMAT
    for off in (0, 8, 12, 13, 16, 24):     # tensor id, K, kind, mode, offset, size
        bd = d.copy(); bd[off] ^= 1
        assert orc.validate(lay.tensors, hdr, bd, p, 7) == O.E_FORMAT, off
    bd = d.copy(); bd[32:64], bd[0:32] = d[0:32], d[32:64]    # order
    assert orc.validate(lay.tensors, hdr, bd, p, 7) == O.E_FORMAT
    e0 = fmt.dirents(d)[0]
    bp = p.copy(); bp[e0["off"]] ^= 1                          # bitmap popcount
    assert orc.validate(lay.tensors, hdr, d, bp, 7) == O.E_FORMAT
    # a DELTA stream is not a retry stream
    W = [x.copy() for x in co]
    assert orc.retry(lay.tensors, W, hdr, d, p, 7) == O.E_FORMAT


def pin_golden_bf16_pairs(orc):
    """Hand-checked BF16 bit patterns (bfloat16 = top 16 bits of IEEE
    binary32) and their masks, from tests/golden/bf16_pairs.txt."""
    rows = []
    with open(os.path.join(GOLDEN, "bf16_pairs.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append([int(x, 16) for x in line.split()])
    old = np.array([r[0] for r in rows], np.uint16)
    new = np.array([r[1] for r in rows], np.uint16)
    mask = np.array([r[2] for r in rows], np.uint32)
    n = len(rows)
    T, S = _one_tensor(n, 2)
    idx, words, (hdr, d, p) = _decode_one(orc, T, S, old, new, n, 2)
    sel = mask != 0
    assert np.array_equal(idx, np.nonzero(sel)[0])
    assert np.array_equal(words, mask[sel])
    W = [old.view(np.uint8).copy()]
    assert orc.apply(T, W, hdr, d, p, np.zeros(len(d) // 32, np.uint8), expected_base_version=0) == 0
    assert np.array_equal(W[0].view(np.uint16), new)


def pin_golden_records(orc):
    """Records worked out by hand from the format definition
    (tests/golden/worked_record_*.txt): a DENSE and a SPARSE high plane."""
    files = sorted(f for f in os.listdir(GOLDEN) if f.startswith("worked_record_"))
    assert len(files) >= 2
    for fn in files:
        spec = {}
        with open(os.path.join(GOLDEN, fn)) as f:
            for line in f:
                line = line.split("#")[0].strip()
                if line:
                    k, v = line.split("=", 1)
                    spec[k.strip()] = v.strip()
        old = np.array([int(x, 16) for x in spec["old"].split()], np.uint16)
        new = np.array([int(x, 16) for x in spec["new"].split()], np.uint16)
        T, S = _one_tensor(len(old), 2)
        rc, hdr, d, p = orc.encode(T, S, [old], [new])
        assert rc == 0
        assert bytes(d).hex() == spec["dirent"].replace(" ", "").lower(), fn
        assert bytes(p).hex() == spec["payload"].replace(" ", "").lower(), fn


def _golden_spec(fn):
    spec = {}
    with open(os.path.join(GOLDEN, fn)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                k, v = line.split("=", 1)
                spec[k.strip()] = v.strip()
    return spec


def pin_golden_header(orc):
    """A 64-byte stream header worked out by hand (tests/golden/worked_header.txt):
    magic, format version, stream kind, chunk size, base and new versions,
    the plan fingerprint (FNV-1a-64 of the serialised tensor table, checked
    against the FNV reference vectors in pin_fingerprint), record and payload
    totals and the zero reserved words, byte for byte."""
    spec = _golden_spec("worked_header.txt")
    src = _golden_spec(spec["source"])
    old = np.array([int(x, 16) for x in src["old"].split()], np.uint16)
    new = np.array([int(x, 16) for x in src["new"].split()], np.uint16)
    T, S = _one_tensor(len(old), 2)
    table = bytes.fromhex(spec["table"])
    assert np.zeros(1, dtype=synth.TENSOR_DT).itemsize == len(table)
    Tb = np.zeros(1, dtype=synth.TENSOR_DT)
    Tb[:] = T
    assert Tb.tobytes() == table
    assert fmt.fnv1a64(table) == int(spec["fingerprint"], 16)
    assert orc.fingerprint(T) == int(spec["fingerprint"], 16)
    rc, hdr, d, p = orc.encode(T, S, [old], [new], base_version=int(spec["base_version"], 16),
                               new_version=int(spec["new_version"], 16))
    assert rc == 0
    assert bytes(hdr).hex() == spec["header"].replace(" ", "").lower()
    assert len(d) == 32 and len(p) == int.from_bytes(bytes(hdr[48:56]), "little")


def pin_group_disjoint_records(orc):
    """The XOR and overwrite records of one chunk may not mark elements of the
    same 16-byte group (the rule that lets apply patch each group with one
    128-bit read-modify-write and keeps records independent, so dedup by
    record id holds: tokendh blog, "XOR or overwrite").  Streams written by
    hand from the format definition: records on different groups of one chunk
    validate and apply element by element; records sharing a group are
    refused by validate, apply and retry, and apply writes nothing."""
    n = 64
    T, S = _one_tensor(n, 2)
    fp = orc.fingerprint(T)
    old = (np.arange(n, dtype=np.uint16) * 0x0101 + 0x3C00).astype(np.uint16)
    # element 0 by XOR mask 0x0001; element 8 (the next group) overwritten
    good = [(0, 0, 0, [0], [0x0001]), (0, 0, 1, [8], [0xBEEF])]
    hdr, d, p = fmt.build_stream(good, 0, 5, 6, fp, [n], [2])
    assert orc.validate(T, hdr, d, p, 5) == 0
    W = [old.view(np.uint8).copy()]
    assert orc.apply(T, W, hdr, d, p, np.zeros(2, np.uint8), expected_base_version=5) == 0
    exp = old.copy()
    exp[0] ^= 0x0001
    exp[8] = 0xBEEF
    assert np.array_equal(W[0].view(np.uint16), exp)
    # the overwrite marks element 7, in the XOR record's group 0..7; and the
    # same clash in a RETRY-kind stream of two overwrite records
    for second in ([7], [3]):
        bad = [(0, 0, 0, [0], [0x0001]), (0, 0, 1, second, [0xBEEF])]
        hdr, d, p = fmt.build_stream(bad, 0, 5, 6, fp, [n], [2])
        assert orc.validate(T, hdr, d, p, 5) == O_E_FORMAT, second
        W = [old.view(np.uint8).copy()]
        assert orc.apply(T, W, hdr, d, p, np.zeros(2, np.uint8), expected_base_version=5) == O_E_FORMAT
        assert np.array_equal(W[0].view(np.uint16), old)
    # group 15..15 of a ragged chunk: elements 56..63 form the last group
    bad = [(0, 0, 0, [63], [0x0100]), (0, 0, 1, [56], [0x1234])]
    hdr, d, p = fmt.build_stream(bad, 0, 5, 6, fp, [n], [2])
    assert orc.validate(T, hdr, d, p, 5) == O_E_FORMAT


def pin_tensor_table_refusals(orc):
    """The oracle refuses tensor tables the format cannot carry (its own
    checks, not the GPU plan builder's): a width other than 1/2/4 bytes, an
    unknown route, XOR routes on 4-byte elements (fp32 tensors go out as
    overwrites), block-scaled tensors without a valid fp32 overwrite scale
    tensor of ceil(numel / block) elements, blocks that split a 16-byte
    group, and scale fields on other routes.  A valid table passes."""
    from oracle import oracle as O

    def table(rows):
        T = np.zeros(len(rows), dtype=synth.TENSOR_DT)
        for i, r in enumerate(rows):
            T[i] = r
        S = np.zeros(len(rows), dtype=synth.SEGMENT_DT)
        for i, r in enumerate(rows):
            S[i]["tensor_id"] = i
            S[i]["shard_id"] = i
            S[i]["ndim"] = 1
            S[i]["extent"] = [int(r[0]), 1, 1, 1]
            S[i]["shard_stride"] = [1, 0, 0, 0]
            S[i]["canon_stride"] = [1, 0, 0, 0]
        return T, S

    def run(rows):
        T, S = table(rows)
        sh = [np.zeros(int(r[0]) * max(int(r[1]), 1), np.uint8) for r in rows]
        rc, *_ = orc.encode(T, S, sh, [x.copy() for x in sh])
        return rc

    ok = [(256, 2, 2, 1, 128), (2, 4, 1, -1, 0)]          # block-scaled BF16 + its fp32 scales
    assert run(ok) == 0
    cases = {
        "width 3": [(16, 3, 1, -1, 0)],
        "route 3": [(16, 2, 3, -1, 0)],
        "XOR on 4-byte": [(16, 4, 0, -1, 0)],
        "block-scaled on 4-byte": [(256, 4, 2, 1, 128), (2, 4, 1, -1, 0)],
        "scale tensor missing": [(256, 2, 2, -1, 128)],
        "scale tensor out of range": [(256, 2, 2, 5, 128), (2, 4, 1, -1, 0)],
        "scale tensor is itself": [(256, 2, 2, 0, 128)],
        "scale tensor not fp32": [(256, 2, 2, 1, 128), (2, 2, 1, -1, 0)],
        "scale tensor not overwrite": [(256, 2, 2, 1, 128), (2, 4, 2, 0, 128)],
        "block of 0": [(256, 2, 2, 1, 0), (2, 4, 1, -1, 0)],
        "block splits a group": [(256, 2, 2, 1, 4), (64, 4, 1, -1, 0)],
        "scale length long": [(256, 2, 2, 1, 128), (3, 4, 1, -1, 0)],
        "scale length short": [(256, 2, 2, 1, 128), (1, 4, 1, -1, 0)],
        "scale fields on affine": [(16, 2, 0, -1, 8)],
        "scale tensor on overwrite": [(16, 2, 1, 0, 0)],
    }
    for name, rows in cases.items():
        assert run(rows) == O.E_INVAL, name
        T, S = table(rows)
        assert orc.validate(T, np.zeros(64, np.uint8), np.zeros(0, np.uint8), np.zeros(0, np.uint8)) == O.E_INVAL, name


def _gaps_stream(orc, idx, n, w=2, mask=0x0001):
    """A one-tensor stream (index-list layout) whose only record changes the
    given elements by `mask`."""
    from oracle import oracle as O
    T, S = _one_tensor(n, w)
    dt = {1: np.uint8, 2: np.uint16}[w]
    old = (0x3C00 + (np.arange(n) % 256)).astype(dt) if w == 2 else (np.arange(n) % 251).astype(dt)
    new = old.copy()
    new[np.asarray(idx, dtype=np.int64)] ^= dt(mask)
    rc, hdr, d, p = orc.encode(T, S, [old], [new], mode=O.MODE_DELTA | O.ENC_LISTS)
    assert rc == 0
    return T, old, new, hdr, d, p


def pin_golden_gaps_record(orc):
    """A packed record worked out by hand (tests/golden/worked_packed_record.txt):
    the index list of 12 changes, and its gap section as unsigned LEB128
    varints, byte for byte; unpacking gives the list record back."""
    from oracle import oracle as O
    spec = _golden_spec("worked_packed_record.txt")
    idx = [int(x) for x in spec["indices"].split()]
    T, old, new, hdr, d, p = _gaps_stream(orc, idx, int(spec["numel"]))
    hx = lambda k: spec[k].replace(" ", "").lower()
    assert bytes(d).hex() == hx("list_dirent") and bytes(p).hex() == hx("list_payload")
    rc, ph, pd, pp = orc.pack_stream(T, hdr, d, p)
    assert rc == 0
    assert bytes(pd).hex() == hx("packed_dirent") and bytes(pp).hex() == hx("packed_payload")
    assert bytes(ph[0:4]).hex() == hx("packed_magic")
    assert int(ph[48:56].view("<u8")[0]) == len(pp) and np.array_equal(ph[4:48], hdr[4:48])
    rc, uh, ud, up = orc.unpack_stream(T, ph, pd, pp)
    assert rc == 0 and np.array_equal(uh, hdr) and np.array_equal(ud, d) and np.array_equal(up, p)
    assert orc.validate(T, ph, pd, pp) == O.E_FORMAT        # a packed stream is not applied as such


def pin_leb128_vectors(orc):
    """Gap varints against hand-derived unsigned LEB128 bytes: one change at
    each of elements 0..7 (eight gaps of 0, one byte each) and then one at
    8 + v, so the ninth varint is v's, for v at the one-, two- and
    three-byte boundaries (uint8 tensor of one 65536-element chunk)."""
    vectors = {0: "00", 1: "01", 127: "7f", 128: "8001", 300: "ac02", 16383: "ff7f", 16384: "808001",
               65527: "f7ff03"}
    for v, hx in vectors.items():
        idx = list(range(8)) + [8 + v]
        T, old, new, hdr, d, p = _gaps_stream(orc, idx, 65536, w=1, mask=0x10)
        rc, ph, pd, pp = orc.pack_stream(T, hdr, d, p)
        assert rc == 0
        assert pd[15] == 2, v                                   # packed: 8 + len(v) bytes < 32
        assert bytes(pp[:8 + len(hx) // 2]).hex() == "00" * 8 + hx, v
        assert not pp[8 + len(hx) // 2:16].any(), v             # zero padding
        assert fmt.leb128(v).hex() == hx


def pin_pack_roundtrip(orc, seeds=range(10)):
    """On random layouts at low change rates with index lists: a list record
    is packed exactly when its padded gap section is strictly smaller than
    its padded list (sizes computed here from the definition); a packed
    record's gap varints decode to the list's indices and its later sections
    are the list record's; unpack(pack(stream)) is the stream, byte for byte;
    the packed stream applies, once unpacked, to new."""
    from oracle import oracle as O
    for seed in seeds:
        lay = synth.random_layout(1900 + seed, rate=[0.002, 0.01, 0.03][seed % 3], max_tensors=5,
                                  max_chunks=4.0)
        olds, news, co, cn = canon_lists(lay)
        for mode in (O.MODE_DELTA, O.MODE_RETRY):
            rc, hdr, d, p = orc.encode(lay.tensors, lay.segments, olds, news, mode=mode | O.ENC_LISTS,
                                       base_version=7, new_version=8)
            assert rc == 0
            rc, ph, pd, pp = orc.pack_stream(lay.tensors, hdr, d, p)
            assert rc == 0
            ents, pents = fmt.dirents(d), fmt.dirents(pd)
            assert len(ents) == len(pents)
            pos = 0
            for e, f in zip(ents, pents):
                assert (e["t"], e["c"], e["K"], e["kind"], e["hi_mode"], e["w"], e["H"]) == \
                       (f["t"], f["c"], f["K"], f["kind"], f["hi_mode"], f["w"], f["H"])
                assert f["off"] == pos
                body = p[e["off"]:e["off"] + e["size"]]
                pbody = pp[f["off"]:f["off"] + f["size"]]
                if e["layout"] == 1:
                    li = body[:2 * e["K"]].view("<u2").astype(np.int64)
                    vb = sum(len(fmt.leb128(int(g))) for g in np.diff(np.concatenate([[-1], li])) - 1)
                    want = fmt.pad16(vb) < fmt.pad16(2 * e["K"])
                    assert (f["layout"] == 2) == want, (seed, e)
                if f["layout"] == 2:
                    gi, used = fmt.read_gaps(pbody, e["K"])
                    assert np.array_equal(gi, body[:2 * e["K"]].view("<u2").astype(np.int64))
                    assert not pbody[used:fmt.pad16(used)].any()
                    assert np.array_equal(pbody[fmt.pad16(used):], body[fmt.pad16(2 * e["K"]):])
                else:
                    assert np.array_equal(pbody, body)
                pos += f["size"]
            assert pos == len(pp)
            rc, uh, ud, up = orc.unpack_stream(lay.tensors, ph, pd, pp)
            assert rc == 0 and np.array_equal(uh, hdr) and np.array_equal(ud, d) and np.array_equal(up, p)


def pin_unpack_refusals(orc):
    """Unpack refuses malformed packed streams: a plain (unpacked) header, a
    nonzero padding byte after the last varint, a varint written longer than
    it needs, a varint cut off by the section's end, an index past the
    chunk's elements, a gap section as long as the list it replaces."""
    from oracle import oracle as O
    spec = _golden_spec("worked_packed_record.txt")
    idx = [int(x) for x in spec["indices"].split()]
    T, old, new, hdr, d, p = _gaps_stream(orc, idx, int(spec["numel"]))
    rc, ph, pd, pp = orc.pack_stream(T, hdr, d, p)
    assert rc == 0
    assert orc.unpack_stream(T, ph, pd, pp)[0] == 0
    bad_h = ph.copy()
    bad_h[0:4] = hdr[0:4]
    assert orc.unpack_stream(T, bad_h, pd, pp)[0] == O.E_FORMAT
    # the golden section uses all 16 bytes; a smaller list leaves padding
    idx2 = [0, 1, 2, 3, 4, 5, 6, 7, 9]
    T2, _o, _n, h2, d2, p2 = _gaps_stream(orc, idx2, 4096)
    rc, ph2, pd2, pp2 = orc.pack_stream(T2, h2, d2, p2)
    assert rc == 0 and pd2[15] == 2 and pp2[9] == 0 and pp2[15] == 0   # 9 one-byte varints, 7 padding bytes
    assert orc.unpack_stream(T2, ph2, pd2, pp2)[0] == 0
    x = pp2.copy(); x[15] = 1                                   # nonzero padding
    assert orc.unpack_stream(T2, ph2, pd2, x)[0] == O.E_FORMAT
    x = pp2.copy(); x[8] |= 0x80; x[9] = 0                      # last varint 01 written as 81 00
    assert orc.unpack_stream(T2, ph2, pd2, x)[0] == O.E_FORMAT
    x = pp2.copy(); x[8:16] = 0x80                             # last varint never ends
    assert orc.unpack_stream(T2, ph2, pd2, x)[0] == O.E_FORMAT
    x = pp.copy(); x[14:16] = [0xB0, 0x10]                      # last gap 2094 -> 2096: index 4097 >= 4096
    assert orc.unpack_stream(T, ph, pd, x)[0] == O.E_FORMAT
    x = pd.copy(); x[24:28] = np.frombuffer(np.uint32(48).tobytes(), np.uint8)   # section as long as the list
    xp = np.concatenate([pp[:16], np.zeros(16, np.uint8), pp[16:]])
    xh = ph.copy(); xh[48:56] = np.frombuffer(np.uint64(48).tobytes(), np.uint8)
    assert orc.unpack_stream(T, xh, x, xp)[0] == O.E_FORMAT


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
