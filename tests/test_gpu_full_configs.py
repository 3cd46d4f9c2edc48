"""Full-size GPU runs of the Llama-8B TP=4, Qwen3-30B-A3B EP=8 (3 %, Beta(2,60)
rates) and block-scaled 5 % hot-row MoE workloads.

  * whole-stream parity: every record of the DELTA and the RETRY stream
    equals, byte for byte, the oracle's record for the same inputs (the
    oracle runs unchanged once per tensor group, on a pool of host threads,
    fed with the device shards copied to host memory); the header and the
    directory's order and contiguous offsets are checked on the whole stream;
  * properties on the whole model: records count exactly the elements whose
    stored bits differ; apply turns the old canonical tensors into the new
    ones; after a kill at 50 % of the records the overwrite retry heals all.
"""
import sys

import numpy as np
import pytest

from bit_exact_xor_amd import dcr, synth
from tests import fmt, stream_check

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def typed(lay, shards):
    """Element-typed views of byte shards (what the layout's assembly expects)."""
    return [x.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[lay.shard_w[s]]) for s, x in enumerate(shards)]


def staged_workspace(plan, sb):
    """The benchmark's launch configuration: a staging area holding every
    chunk's slot (none when device memory is short: in-order look-back)."""
    free, _ = torch.cuda.mem_get_info()
    stage = int(plan.info.max_payload_bytes)
    if stage > int(free) - (4 << 30):
        stage = 0
    say("staging area", f"{stage / 1e9:.2f} GB")
    return dcr.workspace(plan, "cuda", stage)


def run_full(orc, lay, sample_names, partial=False, transcode=False):
    assert torch.cuda.is_available()
    say(lay.name, "plan")
    T = lay.tensors
    plan = dcr.dcr_plan_build(T, [lay.shard_bytes(s) for s in range(lay.n_shards)], lay.segments)
    dcr.dcr_plan_upload(plan, "cuda")
    say(lay.name, "inputs", f"{plan.info.canonical_bytes / 1e9:.1f} GB canonical")
    ob, olds = synth.alloc_shards(lay, "cuda")
    nb, news = synth.alloc_shards(lay, "cuda")
    synth.fill_shards_gpu(lay, olds, 0)
    synth.fill_shards_gpu(lay, news, 1)
    ws = dcr.workspace(plan, "cuda")
    cb = int(plan.info.canonical_bytes)
    sb = dcr.StreamBuffers(plan, "cuda", dir_bytes=2 * 32 * int(plan.info.n_chunks),
                           payload_bytes=int(cb * 0.16) + (1 << 24))
    torch.cuda.synchronize()
    say(lay.name, "encode")
    wss = staged_workspace(plan, sb)
    dcr.dcr_encode(plan, olds, news, 0, 3, 4, sb.header, sb.dir, sb.payload, sb.result, wss)
    torch.cuda.synchronize()
    del wss
    r = sb.result_host()
    assert int(r["status"]) == 0, r
    n_rec, pbytes = int(r["n_records"]), int(r["payload_bytes"])
    # property: records count exactly the differing stored elements
    diff = 0
    for s in range(lay.n_shards):
        w = lay.shard_w[s]
        a = olds[s].view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[w])
        b = news[s].view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[w])
        diff += int((a != b).sum())
    assert int(r["n_changed"]) == diff
    say(lay.name, f"{n_rec} records, {pbytes / 1e9:.2f} GB payload, {diff} changed")

    # the RETRY stream now, so that both streams are checked against the oracle
    rsb = dcr.StreamBuffers(plan, "cuda", dir_bytes=32 * int(plan.info.n_chunks),
                            payload_bytes=int(cb * 0.16) + (1 << 24))
    say(lay.name, "encode RETRY")
    wss = staged_workspace(plan, rsb)
    dcr.dcr_encode(plan, olds, news, 1, 3, 4, rsb.header, rsb.dir, rsb.payload, rsb.result, wss)
    torch.cuda.synchronize()
    del wss
    rr = rsb.result_host()
    assert int(rr["status"]) == 0, rr
    assert int(rr["n_changed"]) == diff

    # whole-stream parity against the oracle
    streams = {0: stream_check.HostStream(sb.header.cpu().numpy(), sb.dir[: n_rec * 32].cpu().numpy(),
                                          sb.payload[:pbytes].cpu().numpy()),
               1: stream_check.HostStream(rsb.header.cpu().numpy(),
                                          rsb.dir[: int(rr["n_records"]) * 32].cpu().numpy(),
                                          rsb.payload[: int(rr["payload_bytes"])].cpu().numpy())}
    for mode, hs in streams.items():
        err = stream_check.check_layout(hs, lay.n_tensors, mode, 3, 4, plan.info.fingerprint)
        assert err is None, (mode, err)
    say(lay.name, f"oracle parity of every record ({stream_check.host_cores()} threads)")
    pr = stream_check.full_parity(orc, lay, olds, news, streams, 3, 4, log=lambda m: say(lay.name, m))
    assert pr["identical"], pr["first_mismatch"]
    assert pr["records"] == n_rec + int(rr["n_records"]) and pr["groups"] > 0
    say(lay.name, f"oracle parity: {pr['records']} records of {pr['groups']} tensor groups identical "
                  f"({pr['seconds']} s)")
    del streams

    # apply / kill at 50 % / retry, on canonical tensors
    co = lay.assemble(typed(lay, olds))
    sizes = [int(T[t]["numel"]) * int(T[t]["elem_bytes"]) for t in range(len(T))]
    offs = np.concatenate([[0], np.cumsum([(s + 255) // 256 * 256 for s in sizes])]).astype(np.int64)
    cbuf = torch.empty(int(offs[-1]), dtype=torch.uint8, device="cuda")
    canon = [cbuf[int(offs[t]):int(offs[t]) + sizes[t]] for t in range(len(T))]
    for t in range(len(T)):
        canon[t].copy_(co[t].reshape(-1).view(torch.uint8))
    del co
    cn = lay.assemble(typed(lay, news))
    hdr = sb.header.cpu().numpy()
    flags = torch.zeros(max(n_rec, 1), dtype=torch.uint8, device="cuda")
    res = torch.zeros(32, dtype=torch.uint8, device="cuda")
    say(lay.name, "apply")
    dcr.dcr_apply(plan, canon, hdr, sb.dir, sb.payload, flags, 0, n_rec, 3, res, ws)
    torch.cuda.synchronize()
    ar = dcr.apply_result(res)
    assert int(ar["n_applied"]) == n_rec and int(ar["n_invalid"]) == 0
    for t in range(len(T)):
        assert torch.equal(canon[t], cn[t].reshape(-1).view(torch.uint8)), lay.tensor_names[t]
    # back to old by re-copying, apply the first half (a kill), retry all
    co = lay.assemble(typed(lay, olds))
    for t in range(len(T)):
        canon[t].copy_(co[t].reshape(-1).view(torch.uint8))
    del co
    flags.zero_()
    dcr.dcr_apply(plan, canon, hdr, sb.dir, sb.payload, flags, 0, n_rec // 2, 3, res, ws)
    if not (partial or transcode):
        del sb
    say(lay.name, "retry")
    if transcode:
        # the same RETRY stream, written from the DELTA stream and old only
        say(lay.name, "retry stream from the DELTA stream")
        tsb = dcr.StreamBuffers(plan, "cuda", dir_bytes=32 * int(plan.info.n_chunks),
                                payload_bytes=int(cb * 0.2) + (1 << 20))
        dcr.dcr_encode_retry_from_delta(plan, olds, hdr, sb.dir, sb.payload, 0, tsb.header, tsb.dir, tsb.payload,
                                        tsb.result, ws)
        torch.cuda.synchronize()
        tr, rr = tsb.result_host(), rsb.result_host()
        assert int(tr["status"]) == 0, tr
        for k in ("n_records", "payload_bytes", "n_changed"):
            assert int(tr[k]) == int(rr[k]), (k, tr, rr)
        nr, pb = int(rr["n_records"]), int(rr["payload_bytes"])
        assert torch.equal(tsb.header, rsb.header)
        assert torch.equal(tsb.dir[: nr * 32], rsb.dir[: nr * 32])
        assert torch.equal(tsb.payload[:pb], rsb.payload[:pb])
        say(lay.name, f"retry stream from the DELTA stream: identical ({nr} records, {pb / 1e9:.2f} GB)")
        del tsb
        if not partial:
            del sb
    dcr.dcr_apply_overwrite_retry(plan, canon, rsb.header.cpu().numpy(), rsb.dir, rsb.payload, 3, res, ws)
    torch.cuda.synchronize()
    for t in range(len(T)):
        assert torch.equal(canon[t], cn[t].reshape(-1).view(torch.uint8)), lay.tensor_names[t]
    say(lay.name, "apply, kill at 50 % and retry: all tensors equal new")
    if partial:
        # again from old, killed at 50 %: the partial retry sends only the
        # chunks of the unflagged records and heals everything
        co = lay.assemble(typed(lay, olds))
        for t in range(len(T)):
            canon[t].copy_(co[t].reshape(-1).view(torch.uint8))
        del co
        flags.zero_()
        dcr.dcr_apply(plan, canon, hdr, sb.dir, sb.payload, flags, 0, n_rec // 2, 3, res, ws)
        say(lay.name, "partial retry")
        wss = staged_workspace(plan, rsb)
        dcr.dcr_encode_retry_partial(plan, olds, news, hdr, sb.dir, flags, 3, 4, rsb.header, rsb.dir, rsb.payload,
                                     rsb.result, wss)
        torch.cuda.synchronize()
        del wss
        pr = rsb.result_host()
        assert int(pr["status"]) == 0, pr
        ents = sb.dir[: n_rec * 32].cpu().numpy().reshape(-1, 32)
        want = sorted(set(zip(ents[n_rec // 2:, 0:4].copy().view("<u4").ravel().tolist(),
                              ents[n_rec // 2:, 4:8].copy().view("<u4").ravel().tolist())))
        pn = int(pr["n_records"])
        pents = rsb.dir[: pn * 32].cpu().numpy().reshape(-1, 32)
        got = list(zip(pents[:, 0:4].copy().view("<u4").ravel().tolist(),
                       pents[:, 4:8].copy().view("<u4").ravel().tolist()))
        assert got == want, (len(got), len(want))
        dcr.dcr_apply_overwrite_retry(plan, canon, rsb.header.cpu().numpy(), rsb.dir, rsb.payload, 3, res, ws)
        torch.cuda.synchronize()
        for t in range(len(T)):
            assert torch.equal(canon[t], cn[t].reshape(-1).view(torch.uint8)), lay.tensor_names[t]
        say(lay.name, f"kill at 50 % and partial retry ({pn} records, {int(pr['payload_bytes']) / 1e9:.2f} GB): "
                      "all tensors equal new")
        del sb
    del cbuf, canon, cn, ob, nb, olds, news, rsb
    torch.cuda.empty_cache()


def test_full_llama8b_receiver_tp2(orc):
    """Config 2 encoded from TP=4 trainer shards, applied straight into a
    receiver that stores the model as TP=2 engine shards (dcr_apply_sharded):
    every tensor read back through the receiver layout equals new, also after
    a kill at 50 % and the overwrite retry into the receiver layout."""
    from tests import gpu_harness as gh
    lay = synth.llama_layout()
    lay_r = synth.llama_layout(tp=2)
    say("cfg2 -> TP=2 receiver", "plans")
    T = lay.tensors
    plan = dcr.dcr_plan_build(T, [lay.shard_bytes(s) for s in range(lay.n_shards)], lay.segments)
    dcr.dcr_plan_upload(plan, "cuda")
    rplan = dcr.dcr_plan_build(lay_r.tensors, [lay_r.shard_bytes(s) for s in range(lay_r.n_shards)], lay_r.segments)
    dcr.dcr_plan_upload(rplan, "cuda")
    assert rplan.info.fingerprint == plan.info.fingerprint
    ob, olds = synth.alloc_shards(lay, "cuda")
    nb, news = synth.alloc_shards(lay, "cuda")
    synth.fill_shards_gpu(lay, olds, 0)
    synth.fill_shards_gpu(lay, news, 1)
    cb = int(plan.info.canonical_bytes)
    sb = dcr.StreamBuffers(plan, "cuda", dir_bytes=2 * 32 * int(plan.info.n_chunks),
                           payload_bytes=int(cb * 0.2) + (1 << 20))
    rsb = dcr.StreamBuffers(plan, "cuda", dir_bytes=32 * int(plan.info.n_chunks),
                            payload_bytes=int(cb * 0.2) + (1 << 20))
    wss = staged_workspace(plan, sb)
    dcr.dcr_encode(plan, olds, news, 0, 3, 4, sb.header, sb.dir, sb.payload, sb.result, wss)
    dcr.dcr_encode(plan, olds, news, 1, 3, 4, rsb.header, rsb.dir, rsb.payload, rsb.result, wss)
    torch.cuda.synchronize()
    del wss
    assert int(sb.result_host()["status"]) == 0 and int(rsb.result_host()["status"]) == 0
    n_rec = sb.n_records()
    hdr, rhdr = sb.header.cpu().numpy(), rsb.header.cpu().numpy()
    co = lay.assemble(typed(lay, olds))
    ws = dcr.workspace(rplan, "cuda")
    res = torch.zeros(32, dtype=torch.uint8, device="cuda")
    flags = torch.zeros(max(n_rec, 1), dtype=torch.uint8, device="cuda")
    for kill in (None, n_rec // 2):
        say("cfg2 -> TP=2 receiver", "apply" if kill is None else "kill at 50 % + retry")
        rbuf, rsh = gh.scatter_shards(lay_r, co)
        flags.zero_()
        dcr.dcr_apply_sharded(rplan, rsh, hdr, sb.dir, sb.payload, flags, 0, n_rec if kill is None else kill, 3,
                              res, ws)
        if kill is not None:
            dcr.dcr_apply_overwrite_retry_sharded(rplan, rsh, rhdr, rsb.dir, rsb.payload, 3, res, ws)
        torch.cuda.synchronize()
        assert int(dcr.apply_result(res)["n_invalid"]) == 0
        got = lay_r.assemble(typed(lay_r, rsh))
        cn = lay.assemble(typed(lay, news))
        for t in range(len(T)):
            assert torch.equal(got[t].reshape(-1), cn[t].reshape(-1)), lay.tensor_names[t]
        del got, cn, rbuf, rsh
        torch.cuda.empty_cache()
    say("cfg2 -> TP=2 receiver: all tensors equal new")


def test_full_llama8b_pipelined():
    """Config 2 through the pipelined transfer: the encode publishes 16
    slices while it runs; each is copied to pinned host memory, back into
    the receiver's buffers and applied with its prefix header on separate
    streams.  The host copy equals the one-shot stream byte for byte, every
    prefix header cuts the stream where the slice rule says, and the
    receiver ends equal to new."""
    from tests import gpu_harness as gh
    from bit_exact_xor_amd.pipeline import HostLoopback
    lay = synth.llama_layout()
    say("cfg2 pipelined", "plan")
    T = lay.tensors
    plan = dcr.dcr_plan_build(T, [lay.shard_bytes(s) for s in range(lay.n_shards)], lay.segments)
    dcr.dcr_plan_upload(plan, "cuda")
    ob, olds = synth.alloc_shards(lay, "cuda")
    nb, news = synth.alloc_shards(lay, "cuda")
    synth.fill_shards_gpu(lay, olds, 0)
    synth.fill_shards_gpu(lay, news, 1)
    cb = int(plan.info.canonical_bytes)
    ref = dcr.StreamBuffers(plan, "cuda", dir_bytes=2 * 32 * int(plan.info.n_chunks),
                            payload_bytes=int(cb * 0.2) + (1 << 20))
    sb = dcr.StreamBuffers(plan, "cuda", dir_bytes=2 * 32 * int(plan.info.n_chunks),
                           payload_bytes=int(cb * 0.2) + (1 << 20))
    wss = staged_workspace(plan, ref)
    dcr.dcr_encode(plan, olds, news, 0, 3, 4, ref.header, ref.dir, ref.payload, ref.result, wss)
    torch.cuda.synchronize()
    r = ref.result_host()
    assert int(r["status"]) == 0
    n_rec, pbytes = int(r["n_records"]), int(r["payload_bytes"])
    co = lay.assemble(typed(lay, olds))
    sizes = [int(T[t]["numel"]) * int(T[t]["elem_bytes"]) for t in range(len(T))]
    offs = np.concatenate([[0], np.cumsum([(s + 255) // 256 * 256 for s in sizes])]).astype(np.int64)
    cbuf = torch.empty(int(offs[-1]), dtype=torch.uint8, device="cuda")
    canon = [cbuf[int(offs[t]):int(offs[t]) + sizes[t]] for t in range(len(T))]
    for t in range(len(T)):
        canon[t].copy_(co[t].reshape(-1).view(torch.uint8))
    del co
    flags = torch.zeros(max(n_rec, 1), dtype=torch.uint8, device="cuda")
    rws = dcr.workspace(plan, "cuda")
    lb = HostLoopback(plan, 32 * n_rec + (1 << 16), pbytes + (1 << 20))
    torch.cuda.synchronize()
    say("cfg2 pipelined", f"encode + transfer + apply, {n_rec} records, {pbytes / 1e9:.2f} GB")
    heads, results = lb.run(olds, news, 0, 3, 4, sb, wss, 16, canon, flags, rws)
    torch.cuda.synchronize()
    assert len(heads) == 16
    assert int(sb.result_host()["status"]) == 0
    ref_hdr = ref.header.cpu().numpy()
    assert np.array_equal(sb.header.cpu().numpy(), ref_hdr) and np.array_equal(heads[-1], ref_hdr)
    ref_dir = ref.dir[: n_rec * 32].cpu()
    assert torch.equal(lb.host_dir[: n_rec * 32], ref_dir)
    assert torch.equal(lb.host_payload[:pbytes], ref.payload[:pbytes].cpu())
    n, pre = gh.expected_prefixes(lay, ref_dir.numpy(), pbytes, 16)
    assert n == 16
    for k, (rk, pk) in enumerate(pre):
        assert int(heads[k][40:48].view("<u8")[0]) == rk and int(heads[k][48:56].view("<u8")[0]) == pk, k
        want = ref_hdr.copy()
        want[40:56] = heads[k][40:56]
        assert np.array_equal(heads[k], want), k
    ar = [dcr.apply_result(x) for x in results]
    assert sum(int(a["n_applied"]) for a in ar) == n_rec and all(int(a["n_invalid"]) == 0 for a in ar)
    cn = lay.assemble(typed(lay, news))
    for t in range(len(T)):
        assert torch.equal(canon[t], cn[t].reshape(-1).view(torch.uint8)), lay.tensor_names[t]
    say("cfg2 pipelined: host copy equals the stream, prefixes cut at the slice ends, receiver equals new")
    del wss, cbuf, canon, cn, ob, nb, olds, news, lb, ref, sb
    torch.cuda.empty_cache()


def test_full_llama8b_tp4(orc):
    lay = synth.llama_layout()
    run_full(orc, lay, ["model.layers.0.input_layernorm.weight", "model.layers.0.self_attn.q_proj.weight",
                        "model.layers.0.self_attn.k_proj.weight", "model.layers.0.self_attn.o_proj.weight",
                        "model.layers.31.mlp.down_proj.weight", "model.norm.weight"], partial=True,
             transcode=True)


def test_full_qwen30b_ep8_beta(orc):
    lay = synth.config3_layout()
    run_full(orc, lay, ["model.layers.0.self_attn.q_proj.weight", "model.layers.0.self_attn.o_proj.weight",
                        "model.layers.0.mlp.gate.weight", "model.layers.0.self_attn.q_norm.weight",
                        "model.layers.0.mlp.experts.0.gate_proj.weight",
                        "model.layers.47.mlp.experts.127.down_proj.weight", "model.norm.weight"])


def test_full_qwen30b_hot_block_scaled(orc):
    lay = synth.config4_layout()
    run_full(orc, lay, ["model.layers.0.self_attn.q_proj.weight", "model.layers.0.mlp.gate.weight",
                        "model.layers.0.mlp.experts.0.gate_proj.weight",
                        "model.layers.0.mlp.experts.5.down_proj.weight",
                        "model.layers.47.mlp.experts.127.up_proj.weight", "model.norm.weight"], transcode=True)
