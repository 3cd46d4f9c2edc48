"""Host-side checks of libdcr.so (no GPU): symbols, constants, plan building."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from bit_exact_xor_amd import dcr, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "dcr.h")).read()
    return sorted(set(re.findall(r"\b(dcr_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = dcr.load_library()
    names = declared_symbols()
    assert {"dcr_plan_build", "dcr_encode", "dcr_apply", "dcr_apply_overwrite_retry"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", dcr.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (dcr_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_format_constants_agree_with_oracle():
    from oracle import oracle as O
    c = dcr.format_constants()
    assert c == [0x31524344, 1, O.CHUNK_BYTES, O.HEADER_BYTES, O.DIRENT_BYTES,
                 O.ORC_TENSOR.itemsize, O.ORC_SEGMENT.itemsize, 64, O.ENC_LISTS, O.LAYOUT_LIST]
    assert dcr.TENSOR_DESC == O.ORC_TENSOR or dcr.TENSOR_DESC.descr == O.ORC_TENSOR.descr
    assert dcr.SEGMENT.itemsize == O.ORC_SEGMENT.itemsize


def test_plan_fingerprint_matches_oracle(orc):
    for seed in range(5):
        lay = synth.random_layout(seed)
        p = dcr.dcr_plan_build(lay.tensors, [lay.shard_bytes(s) for s in range(lay.n_shards)], lay.segments)
        assert p.info.fingerprint == orc.fingerprint(lay.tensors)
        assert p.info.canonical_bytes == lay.total_bytes()


def test_plan_pieces_llama_tp4():
    lay = synth.llama_layout(hidden=256, layers=2, ffn=640, n_q=8, n_kv=4, head_dim=32, vocab=1000, tp=4)
    p = dcr.dcr_plan_build(lay.tensors, [lay.shard_bytes(s) for s in range(lay.n_shards)], lay.segments)
    n_chunks = sum(-(-int(t["numel"]) * 2 // 65536) for t in lay.tensors)
    assert p.info.n_chunks == n_chunks
    assert p.info.n_pieces > n_chunks  # row-parallel o / down tensors split chunks into runs


def test_plan_rejects_bad_layouts():
    T = np.zeros(1, dtype=synth.TENSOR_DT)
    T[0] = (100, 2, 0, -1, 0)
    S = np.zeros(2, dtype=synth.SEGMENT_DT)
    for i in range(2):
        S[i]["ndim"] = 1
        S[i]["shard_stride"][0] = 1
        S[i]["canon_stride"][0] = 1
    S[0]["extent"][0], S[1]["extent"][0] = 60, 40
    S[1]["shard_off"], S[1]["canon_off"] = 60, 60
    dcr.dcr_plan_build(T, [200], S)                     # exact cover
    S2 = S.copy(); S2[1]["canon_off"] = 59                # overlap + gap
    with pytest.raises(dcr.DcrError) as e:
        dcr.dcr_plan_build(T, [200], S2)
    assert e.value.code == dcr.DCR_E_COVERAGE
    S2 = S.copy(); S2[1]["extent"][0] = 39                # gap at the end
    with pytest.raises(dcr.DcrError) as e:
        dcr.dcr_plan_build(T, [200], S2)
    assert e.value.code == dcr.DCR_E_COVERAGE
    S2 = S.copy(); S2[1]["shard_off"] = 170               # shard overrun
    with pytest.raises(dcr.DcrError) as e:
        dcr.dcr_plan_build(T, [200], S2)
    assert e.value.code == dcr.DCR_E_INVAL
    T2 = T.copy(); T2[0]["elem_bytes"] = 4                # XOR route on 4-byte elements
    with pytest.raises(dcr.DcrError) as e:
        dcr.dcr_plan_build(T2, [400], S)
    assert e.value.code == dcr.DCR_E_INVAL
    T3 = T.copy(); T3[0]["route"] = 2                     # block-scaled without scales
    with pytest.raises(dcr.DcrError):
        dcr.dcr_plan_build(T3, [200], S)


def test_plan_accepts_degenerate_tensors():
    T = np.zeros(3, dtype=synth.TENSOR_DT)
    T[0] = (0, 2, 0, -1, 0)
    T[1] = (1, 1, 1, -1, 0)
    T[2] = (7, 2, 0, -1, 0)
    S = np.zeros(2, dtype=synth.SEGMENT_DT)
    S[0] = (1, 0, 1, 0, 0, 0, [1, 1, 1, 1], [1, 0, 0, 0], [1, 0, 0, 0])
    S[1] = (2, 1, 1, 0, 0, 0, [7, 1, 1, 1], [1, 0, 0, 0], [1, 0, 0, 0])
    p = dcr.dcr_plan_build(T, [1, 14], S)
    assert p.info.n_chunks == 2


def test_ready_wait_host_logic():
    """dcr_ready_wait only reads host memory: published count, failure status
    and the prefix headers of a watermark region (no GPU involved)."""
    n = 3
    r = np.zeros(dcr.ready_region_bytes(n) + 64, dtype=np.uint8)
    reg = r[(-r.ctypes.data) % 64:][: dcr.ready_region_bytes(n)]   # 64-byte aligned view
    assert reg.ctypes.data % 64 == 0
    reg[12:16] = np.frombuffer(np.uint32(n).tobytes(), np.uint8)
    for k in range(n):
        reg[64 + 64 * k: 128 + 64 * k] = np.arange(64, dtype=np.uint8) + 16 * k
    with pytest.raises(dcr.DcrError) as e:
        dcr.dcr_ready_wait(reg, 0, timeout_us=2000)
    assert e.value.code == dcr.DCR_E_TIMEOUT
    reg[0:8] = np.frombuffer(np.uint64(2).tobytes(), np.uint8)
    assert np.array_equal(dcr.dcr_ready_wait(reg, 0, 1000), np.arange(64, dtype=np.uint8))
    assert np.array_equal(dcr.dcr_ready_wait(reg, 1, 1000), np.arange(64, dtype=np.uint8) + 16)
    with pytest.raises(dcr.DcrError) as e:
        dcr.dcr_ready_wait(reg, 2, timeout_us=2000)
    assert e.value.code == dcr.DCR_E_TIMEOUT
    reg[8:12] = np.frombuffer(np.int32(dcr.DCR_E_CAPACITY).tobytes(), np.uint8)
    with pytest.raises(dcr.DcrError) as e:
        dcr.dcr_ready_wait(reg, 2, timeout_us=10_000_000)
    assert e.value.code == dcr.DCR_E_CAPACITY
    assert np.array_equal(dcr.dcr_ready_wait(reg, 1, 0), np.arange(64, dtype=np.uint8) + 16)
    with pytest.raises(dcr.DcrError) as e:
        dcr.dcr_ready_wait(reg, 3, timeout_us=1000)
    assert e.value.code == dcr.DCR_E_INVAL


def test_compact_stage_bytes():
    """max_payload_bytes is every chunk's worst-case records (one 4096x4096
    BF16 tensor: 512 full chunks, each at most a 4 KiB bitmap plus two 32 KiB
    planes, 512 x 69 632 bytes); compact_stage_bytes is 1/16 of it, 16-byte
    aligned, and never below 1 KiB (16 bytes for each of 64 partitions)."""
    from bit_exact_xor_amd import dcr, synth
    lay = synth.config1_layout()
    plan = dcr.dcr_plan_build(lay.tensors, [lay.shard_bytes(s) for s in range(lay.n_shards)], lay.segments)
    assert plan.info.n_chunks == 512
    assert plan.info.max_payload_bytes == 512 * (4096 + 2 * 32768)
    assert plan.info.compact_stage_bytes == 32 * (4096 + 2 * 32768)
    small = synth.config1_layout(40, 40)
    p2 = dcr.dcr_plan_build(small.tensors, [small.shard_bytes(s) for s in range(small.n_shards)], small.segments)
    assert p2.info.n_chunks == 1
    # 1600 elements: 208-byte bitmap, two 1600-byte planes -> 3408; /16 = 213
    assert p2.info.max_payload_bytes == 3408
    assert p2.info.compact_stage_bytes == 1024


def test_plan_chunk_limit():
    """A plan holds at most (2^32 - 1) / 1024 chunks, since the encode runs one
    1024-thread workgroup per chunk in one grid: one uint8 tensor of exactly
    that many 64 KiB chunks builds, one more chunk is refused (no memory is
    touched: sizes only, the plan tables are a few dozen bytes per chunk)."""
    limit = (2 ** 32 - 1) // 1024
    for n_chunks, ok in ((limit, True), (limit + 1, False)):
        numel = n_chunks * 65536
        T = np.zeros(1, dtype=synth.TENSOR_DT)
        T[0] = (numel, 1, 1, -1, 0)
        S = np.zeros(1, dtype=synth.SEGMENT_DT)
        S[0] = (0, 0, 1, 0, 0, 0, [numel, 1, 1, 1], [1, 0, 0, 0], [1, 0, 0, 0])
        if ok:
            p = dcr.dcr_plan_build(T, [numel], S)
            assert p.info.n_chunks == limit
            del p
        else:
            with pytest.raises(dcr.DcrError) as e:
                dcr.dcr_plan_build(T, [numel], S)
            assert e.value.code == dcr.DCR_E_INVAL


def test_encode_noalloc_refuses_large_workspace():
    """dcr_encode_noalloc refuses, before any device work, a plan whose
    workspace exceeds the library's scratch array (DCR_E_CAPACITY); a plan
    of 3 M chunks needs about 80 MB of workspace against 64 MiB."""
    n_chunks = 3_000_000
    numel = n_chunks * 65536
    T = np.zeros(1, dtype=synth.TENSOR_DT)
    T[0] = (numel, 1, 1, -1, 0)
    S = np.zeros(1, dtype=synth.SEGMENT_DT)
    S[0] = (0, 0, 1, 0, 0, 0, [numel, 1, 1, 1], [1, 0, 0, 0], [1, 0, 0, 0])
    p = dcr.dcr_plan_build(T, [numel], S)
    assert p.info.workspace_bytes > dcr.NOALLOC_SCRATCH_BYTES
    with pytest.raises(dcr.DcrError) as e:
        dcr.dcr_encode_noalloc(p, [0x1000], [0x1000], 0, 0, 1, 0x1000, 0x1000, 0x1000, 0x1000, stream=1)
    assert e.value.code == dcr.DCR_E_CAPACITY
    assert "scratch" in str(e.value)
