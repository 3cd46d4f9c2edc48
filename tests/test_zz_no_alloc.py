"""The allocation-free encode (dcr_encode_noalloc) against dcr_encode.

dcr_encode_noalloc runs the encode with the library's own device scratch
array as its workspace.  Two calls in a row through the C-ABI, the second on
a smaller input: a scaled Llama TP=4 layout too large to stage in the array
(so it runs in order) and then a small one that stages whole.  Each stream,
DELTA and RETRY, must equal the stream dcr_encode writes with a workspace of
its own (a full staging area), byte for byte, and every record must equal
the oracle's.  The output buffers are filled with a poison byte first, so
nothing left over passes.
"""
import sys

import numpy as np
import pytest

from bit_exact_xor_amd import dcr, synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


LAYOUTS = [
    ("llama hidden 2048, 4 layers, TP=4 (in order in the scratch array)",
     dict(hidden=2048, layers=4, ffn=5632, n_q=16, n_kv=4, head_dim=128, vocab=32000, tp=4)),
    ("llama hidden 256, 2 layers, TP=4 (staged in the scratch array)",
     dict(hidden=256, layers=2, ffn=640, n_q=8, n_kv=4, head_dim=32, vocab=1000, tp=4)),
]


def test_encode_noalloc_matches_encode(orc):
    from tests import gpu_harness as gh
    from tests import stream_check as sc
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dcr.load_library()
    for name, kw in LAYOUTS:
        lay = synth.llama_layout(**kw, seed=0xDC20A110)
        say("noalloc", name)
        g = gh.Gpu(lay, gen_gpu=True)
        info = g.plan.info
        staged = int(info.workspace_bytes) + int(info.max_payload_bytes) <= dcr.NOALLOC_SCRATCH_BYTES
        assert staged == ("staged" in name), (int(info.workspace_bytes), int(info.max_payload_bytes))
        streams = {}
        for mode in (dcr.MODE_DELTA, dcr.MODE_RETRY):
            ref = g.encode(mode, base=11, new=12, stage=int(info.max_payload_bytes))
            sb = dcr.StreamBuffers(g.plan, "cuda")
            for t in (sb.header, sb.dir, sb.payload, sb.result):
                t.fill_(0xA5)
            dcr.dcr_encode_noalloc(g.plan, g.olds, g.news, mode, 11, 12, sb.header, sb.dir, sb.payload, sb.result)
            torch.cuda.synchronize()
            r, rr = sb.result_host(), ref.result_host()
            assert int(r["status"]) == 0, r
            for k in ("n_records", "payload_bytes", "n_changed", "status"):
                assert int(r[k]) == int(rr[k]), (mode, k, r, rr)
            n, pb = int(r["n_records"]), int(r["payload_bytes"])
            assert n > 0
            assert torch.equal(sb.header, ref.header), mode
            assert torch.equal(sb.dir[: 32 * n], ref.dir[: 32 * n]), mode
            assert torch.equal(sb.payload[:pb], ref.payload[:pb]), mode
            streams[mode] = sc.HostStream(sb.header.cpu().numpy(), sb.dir[: 32 * n].cpu().numpy(),
                                          sb.payload[:pb].cpu().numpy())
            assert sc.check_layout(streams[mode], lay.n_tensors, mode, 11, 12, int(info.fingerprint)) is None
            say("noalloc", name, f"mode {mode}: {n} records, {pb} bytes, equal to dcr_encode")
        pr = sc.full_parity(orc, lay, g.olds, g.news, streams, 11, 12)
        assert pr["identical"], pr["first_mismatch"]
        say("noalloc", name, f"every record equal to the oracle's ({pr['records']} records)")
        del g
        torch.cuda.empty_cache()
