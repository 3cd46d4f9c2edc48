"""CPU checks of bench.py's measurement helpers (no GPU): the touched
16-byte groups, 32-byte sectors and 128-byte lines that price an apply, and
the per-group bit array the read-modify-write ceiling probe patches."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")


def test_touched_counts_and_bits():
    import bench
    rng = np.random.default_rng(3)
    n_bytes = 1 << 14
    old = rng.integers(0, 256, n_bytes, dtype=np.uint8)
    new = old.copy()
    idx = rng.choice(n_bytes, 300, replace=False)
    new[idx] ^= rng.integers(1, 256, 300, dtype=np.uint8)
    o, n = torch.from_numpy(old), torch.from_numpy(new)
    # two tensors at 128-byte aligned offsets of one flat buffer, the second
    # with a ragged end (not a whole line)
    spans = [(0, 4096), (4096, n_bytes - 4096 - 48)]
    gb = torch.zeros(n_bytes // 16 // 8, dtype=torch.uint8)
    g, s, l = bench._touched([o[a:a + m] for a, m in spans], [n[a:a + m] for a, m in spans], gb,
                             [a for a, _ in spans])
    d = np.zeros(n_bytes, bool)
    for a, m in spans:
        d[a:a + m] = old[a:a + m] != new[a:a + m]
    exp_groups = d.reshape(-1, 16).any(1)
    assert g == int(exp_groups.sum())
    assert s == int(d.reshape(-1, 32).any(1).sum())
    assert l == int(d.reshape(-1, 128).any(1).sum())
    bits = np.unpackbits(gb.numpy(), bitorder="little").astype(bool)
    assert np.array_equal(bits, exp_groups)


def test_touched_rejects_unaligned_offsets():
    import bench
    x = torch.zeros(32, dtype=torch.uint8)
    with pytest.raises(AssertionError):
        bench._touched([x], [x], torch.zeros(4, dtype=torch.uint8), [16])


def test_source_hash_ignores_comments_only(tmp_path):
    """The hash that ties a committed counter summary to the kernel sources:
    unchanged by comment and layout edits, changed by any edit to the code."""
    import bench
    base = "// header\nint f(int x) { /* note */ return x + 1; }  // tail\n"
    p = tmp_path / "k.hip"
    p.write_text(base)
    h0 = bench._src_sha256([str(p)])
    p.write_text("// other header\n\nint f(int x) {\n    /* changed note */\n    return x + 1;\n}\n")
    assert bench._src_sha256([str(p)]) == h0
    p.write_text(base.replace("x + 1", "x + 2"))
    assert bench._src_sha256([str(p)]) != h0
    assert bench._code_text(base) == "int f(int x) { return x + 1; }"
