"""Seeded synthetic inputs: trainer layouts and BF16 / uint8 / fp32 shard contents.

This module is the one thing both sides share (the GPU library's tests and
benchmark, and the CPU oracle): it describes the inputs and nothing of the
method -- no bit comparison, no projection walk, no record logic.

Random numbers come from a counter-based generator: the i-th output of a
SplitMix64 sequence (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), ``mix64(key + (i + 1) * GAMMA)``, so any
element of any shard can be regenerated on its own, here in numpy or on the
GPU by ``csrc/synth.hip``, which implements the same definition and must
produce the same bits.

Value recipes (all integer except one fp32 multiply and one fp32 add, each a
single correctly rounded IEEE operation, so the CPU and GPU agree bit for bit):

* BF16 "old" weights ~ N(0, 0.02): Irwin-Hall sum of the four 16-bit lanes of
  one 64-bit hash (a bell curve with the right mean and spread), times one
  fp32 constant, rounded to BF16 by round-to-nearest-even on the integer bits.
* a changed BF16 element moves to a neighbouring BF16 value (one unit in the
  last place, random direction, never to Inf/NaN); element i changes iff the
  low 32 bits of its change hash are below ``thr`` (Bernoulli(thr / 2**32)).
* uint8 (NVFP4-packed) bytes: uniform; a change replaces one random nibble by
  a different 4-bit code.
* fp32 scales: positive normal floats; a changed block gets different bits.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable

import numpy as np

M64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
# sd of the sum of four uniform 16-bit integers: sqrt((65536**2 - 1) / 3)
_IH_SD = math.sqrt((65536.0 ** 2 - 1.0) / 3.0)
SCALE_F32 = np.float32(0.02 / _IH_SD)
SCALE_BITS = int(SCALE_F32.view(np.uint32))

# kinds of generated regions
GEN_BF16 = 0      # BF16 N(0,0.02), +-1 ulp changes
GEN_U8 = 1        # uint8 nibble codes, one-nibble changes
GEN_F32SCALE = 2  # fp32 positive scales, changes flagged per element
GEN_BF16_HOT = 3  # like GEN_BF16, plus: listed hot rows change with certainty, and
                  # whole blocks change when their (coupled) scale changes

# neutral descriptions of the plan inputs (each side packs its own struct)
TENSOR_DT = np.dtype([("numel", "<u8"), ("elem_bytes", "<u4"), ("route", "<u4"),
                      ("scale_tensor", "<i4"), ("scale_block", "<u4")])
SEGMENT_DT = np.dtype([("tensor_id", "<u4"), ("shard_id", "<u4"), ("ndim", "<u4"),
                       ("reserved", "<u4"), ("shard_off", "<u8"), ("canon_off", "<u8"),
                       ("extent", "<u8", (4,)), ("shard_stride", "<i8", (4,)),
                       ("canon_stride", "<i8", (4,))])
ROUTE_AFFINE_XOR, ROUTE_OVERWRITE, ROUTE_BLOCK_SCALED = 0, 1, 2


# ------------------------------------------------------------- the generator

def mix64(z):
    """SplitMix64 output mix on uint64 numpy arrays (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        z = z ^ (z >> np.uint64(31))
    return z


def mix64_int(z: int) -> int:
    z &= M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def derive_key(seed: int, stream: int, purpose: int) -> int:
    """Key of one generated stream: SplitMix64 output number 2*stream+purpose."""
    return mix64_int(seed + GAMMA * (2 * stream + purpose + 1))


def hashes(key: int, start: int, n: int) -> np.ndarray:
    """Outputs start .. start+n-1 of the SplitMix64 sequence with state key."""
    i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(np.uint64(key) + i * np.uint64(GAMMA))


def f32_to_bf16_rne(f: np.ndarray) -> np.ndarray:
    b = np.asarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_old(key_old: int, start: int, n: int) -> np.ndarray:
    h = hashes(key_old, start, n)
    s = ((h & 0xFFFF) + ((h >> 16) & 0xFFFF) + ((h >> 32) & 0xFFFF) + (h >> 48)).astype(np.int64)
    x = (s - 131070).astype(np.float32)          # exact: |x| < 2**24
    return f32_to_bf16_rne(x * SCALE_F32)        # one fp32 multiply, then RNE


def bf16_step(old: np.ndarray, up: np.ndarray) -> np.ndarray:
    """Neighbouring BF16 value: magnitude +-1 ulp (zero goes to the smallest subnormal)."""
    o = old.astype(np.uint32)
    mag = o & 0x7FFF
    new = np.where(mag == 0, o | 1,
                   np.where(up & (mag < 0x7F7F), o + 1, o - 1))
    return new.astype(np.uint16)


def change_mask(key_chg: int, start: int, n: int, thr: int):
    """(changed, up) for elements start..start+n-1: changed iff low32(hash) < thr."""
    h = hashes(key_chg, start, n)
    changed = (h & np.uint64(0xFFFFFFFF)) < np.uint64(thr)
    up = ((h >> np.uint64(32)) & np.uint64(1)).astype(bool)
    return changed, up, h


def gen_region(kind: int, key_old: int, key_chg: int, thr: int, start: int, n: int,
               version: int, row_len: int = 0, hot_rows: np.ndarray | None = None,
               key_blk: int = 0, thr_blk: int = 0, blk: int = 0) -> np.ndarray:
    """Contents of elements start..start+n-1 of one region, version 0 (old) or 1 (new)."""
    if kind in (GEN_BF16, GEN_BF16_HOT):
        old = bf16_old(key_old, start, n)
        if version == 0:
            return old
        changed, up, _ = change_mask(key_chg, start, n, thr)
        if kind == GEN_BF16_HOT and hot_rows is not None and len(hot_rows):
            rows = (np.arange(start, start + n, dtype=np.int64) // row_len)
            changed = changed | np.isin(rows, hot_rows)
        if kind == GEN_BF16_HOT and blk:
            b0, b1 = start // blk, (start + n - 1) // blk
            bch, _u, _h = change_mask(key_blk, b0, b1 - b0 + 1, thr_blk)
            changed = changed | bch[np.arange(start, start + n, dtype=np.int64) // blk - b0]
        return np.where(changed, bf16_step(old, up), old).astype(np.uint16)
    if kind == GEN_U8:
        old = (hashes(key_old, start, n) & np.uint64(0xFF)).astype(np.uint8)
        if version == 0:
            return old
        changed, _, h = change_mask(key_chg, start, n, thr)
        shift = ((h >> np.uint64(33)) & np.uint64(1)) * np.uint64(4)
        nib = (old.astype(np.uint64) >> shift) & np.uint64(0xF)
        newnib = (nib + np.uint64(1) + ((h >> np.uint64(34)) % np.uint64(15))) & np.uint64(0xF)
        new = (old.astype(np.uint64) & ~(np.uint64(0xF) << shift)) | (newnib << shift)
        return np.where(changed, new.astype(np.uint8), old)
    if kind == GEN_F32SCALE:
        h = hashes(key_old, start, n)
        old = (np.uint64(0x3B000000) + (h & np.uint64(0x00FFFFFF))).astype(np.uint32)
        if version == 0:
            return old
        changed, _, hc = change_mask(key_chg, start, n, thr)
        new = old ^ (np.uint32(1) + ((hc >> np.uint64(40)) & np.uint64(0x3FF)).astype(np.uint32))
        return np.where(changed, new, old).astype(np.uint32)
    raise ValueError(kind)


# --------------------------------------------------------------- layouts

@dataclasses.dataclass
class Region:
    """Elements [elem_off, elem_off+n) of a shard are generated as one stream."""
    shard: int
    elem_off: int
    n: int
    kind: int
    key_old: int
    key_chg: int
    thr: int
    row_len: int = 0
    hot_rows: np.ndarray | None = None
    key_blk: int = 0       # GEN_BF16_HOT: change key of the coupled scale region
    thr_blk: int = 0
    blk: int = 0           # elements per coupled block (0: none)


@dataclasses.dataclass
class Layout:
    name: str
    tensor_names: list
    tensors: np.ndarray            # TENSOR_DT
    segments: np.ndarray           # SEGMENT_DT
    shard_elems: list              # elements per shard
    shard_w: list                  # element bytes per shard
    regions: list                  # Region
    assemble: Callable | None = None  # shards (list of tensors) -> canonical tensors (library ops)
    meta: dict = dataclasses.field(default_factory=dict)
    values: tuple | None = None    # explicit (old_shards, new_shards) numpy lists, if not generated

    @property
    def n_tensors(self):
        return len(self.tensors)

    @property
    def n_shards(self):
        return len(self.shard_elems)

    def shard_bytes(self, s):
        return self.shard_elems[s] * self.shard_w[s]

    def total_bytes(self):
        return int(sum(int(t["numel"]) * int(t["elem_bytes"]) for t in self.tensors))

    def shard_host(self, s: int, version: int) -> np.ndarray:
        """Generate one shard's contents in numpy (element dtype)."""
        if self.values is not None:
            return self.values[version][s]
        w = self.shard_w[s]
        dt = {1: np.uint8, 2: np.uint16, 4: np.uint32}[w]
        out = np.zeros(self.shard_elems[s], dtype=dt)
        for r in self.regions:
            if r.shard != s:
                continue
            out[r.elem_off:r.elem_off + r.n] = gen_region(
                r.kind, r.key_old, r.key_chg, r.thr, 0, r.n, version, r.row_len, r.hot_rows,
                r.key_blk, r.thr_blk, r.blk)
        return out

    def shards_host(self, version: int) -> list:
        return [self.shard_host(s, version) for s in range(self.n_shards)]


class _Builder:
    def __init__(self, name, seed):
        self.name, self.seed = name, seed
        self.tnames, self.tensors, self.segs = [], [], []
        self.shard_elems, self.shard_w, self.regions = [], [], []
        self._stream = 0

    def tensor(self, name, numel, w, route=ROUTE_AFFINE_XOR, scale_tensor=-1, scale_block=0):
        self.tnames.append(name)
        self.tensors.append((numel, w, route, scale_tensor, scale_block))
        return len(self.tensors) - 1

    def shard(self, n_elems, w):
        self.shard_elems.append(int(n_elems))
        self.shard_w.append(int(w))
        return len(self.shard_elems) - 1

    def seg(self, t, s, shard_off, canon_off, extent, shard_stride, canon_stride):
        nd = len(extent)
        ext = list(extent) + [1] * (4 - nd)
        ss = list(shard_stride) + [0] * (4 - nd)
        cs = list(canon_stride) + [0] * (4 - nd)
        self.segs.append((t, s, nd, 0, shard_off, canon_off, ext, ss, cs))

    def region(self, shard, elem_off, n, kind, thr, row_len=0, hot_rows=None, key_chg=None,
               key_blk=0, thr_blk=0, blk=0):
        sid = self._stream
        self._stream += 1
        kc = derive_key(self.seed, sid, 1) if key_chg is None else key_chg
        self.regions.append(Region(shard, elem_off, n, kind, derive_key(self.seed, sid, 0),
                                   kc, int(thr), row_len, hot_rows, key_blk, int(thr_blk), blk))
        return self.regions[-1]

    def build(self, assemble=None, meta=None) -> Layout:
        T = np.zeros(len(self.tensors), dtype=TENSOR_DT)
        for i, (numel, w, route, st, sb) in enumerate(self.tensors):
            T[i] = (numel, w, route, st, sb)
        S = np.zeros(len(self.segs), dtype=SEGMENT_DT)
        for i, (t, s, nd, _r, so, co, ext, ss, cs) in enumerate(self.segs):
            S[i]["tensor_id"], S[i]["shard_id"], S[i]["ndim"] = t, s, nd
            S[i]["shard_off"], S[i]["canon_off"] = so, co
            S[i]["extent"], S[i]["shard_stride"], S[i]["canon_stride"] = ext, ss, cs
        return Layout(self.name, self.tnames, T, S, self.shard_elems, self.shard_w,
                      self.regions, assemble, meta or {})


def rate_thr(rate: float) -> int:
    return int(min(max(round(rate * 2.0 ** 32), 0), 1 << 32))


# ---------------------------------------------------------------- config 1

def config1_layout(n_rows=4096, n_cols=4096, seed=0xDC202601) -> Layout:
    """One [4096,4096] BF16 tensor, one shard, identity projection, all XOR."""
    b = _Builder("cfg1", seed)
    t = b.tensor("weight", n_rows * n_cols, 2)
    s = b.shard(n_rows * n_cols, 2)
    b.seg(t, s, 0, 0, [n_rows * n_cols], [1], [1])
    lay = b.build(assemble=lambda sh: [sh[0].reshape(-1)],
                  meta={"seed": seed, "shape": (n_rows, n_cols)})
    return lay


def config1_values(lay: Layout, lr: float | None = None, target=0.01, n_flips=64):
    """Old / new for config 1: new = BF16(fp32(old) + lr*s), s a signed noise
    uniform in (-1, 1), plus forced +0 <-> -0 flips.  With lr given, that value
    is used; otherwise lr is found by bisection so that the changed fraction
    (flips included) lands within 0.5 % (relative) of target."""
    seed = lay.meta["seed"]
    n = int(lay.tensors[0]["numel"])
    key_old, key_sgn, key_flip = (derive_key(seed, 0, 0), derive_key(seed, 0, 1),
                                  derive_key(seed, 1, 0))
    old = bf16_old(key_old, 0, n)
    u23 = (hashes(key_sgn, 0, n) >> np.uint64(41)).astype(np.int64)       # [0, 2**23)
    s = ((2 * u23 + 1 - (1 << 23)).astype(np.float32)) / np.float32(1 << 23)  # exact
    f_old = (old.astype(np.uint32) << 16).view(np.float32)
    # distinct flip positions from the hash sequence
    pos, i = [], 0
    seen = set()
    while len(pos) < n_flips:
        p = int(hashes(key_flip, i, 1)[0] % np.uint64(n))
        i += 1
        if p not in seen:
            seen.add(p)
            pos.append(p)
    pos = np.array(pos, dtype=np.int64)

    def make(lr_):
        new = f32_to_bf16_rne(f_old + np.float32(lr_) * s)
        o2, n2 = old.copy(), new
        o2[pos[:n_flips // 2]], n2[pos[:n_flips // 2]] = 0x0000, 0x8000
        o2[pos[n_flips // 2:]], n2[pos[n_flips // 2:]] = 0x8000, 0x0000
        return o2, n2

    if lr is None:
        lo, hi = 0.0, 1e-4
        for _ in range(80):
            mid = float(np.float32(0.5 * (lo + hi)))
            o2, n2 = make(mid)
            frac = float(np.count_nonzero(o2 != n2)) / n
            if abs(frac - target) <= target * 0.005:
                lr = mid
                break
            if frac < target:
                lo = mid
            else:
                hi = mid
        else:
            lr = float(np.float32(0.5 * (lo + hi)))
    o2, n2 = make(lr)
    return o2, n2, float(lr), pos


# ------------------------------------------------------- config 2 (Llama)

def llama_layout(hidden=4096, layers=32, ffn=14336, n_q=32, n_kv=8, head_dim=128,
                 vocab=128256, tp=4, rate=0.01, seed=0xDC202602, name="cfg2", gate_up_group=0) -> Layout:
    """Llama-style dense checkpoint trained with tensor parallelism tp.

    Trainer shards per rank r: vocab-parallel embed / lm_head rows; a fused
    QKV [groups x (q_per_group + 2) x head_dim, hidden] (route OVERWRITE in
    canonical q/k/v); o_proj row-parallel (input columns split); fused fc1
    [gate_r ; up_r] (output rows split); down_proj row-parallel.  Norms are
    replicated; rank 0 owns them (other replicas are never read).

    gate_up_group > 0: the fused fc1 of each rank interleaves gate and up
    rows in groups of that many rows ([gate 0..g-1, up 0..g-1, gate g..2g-1,
    ...]), the physical layout a fused MoE / MLP kernel may want (the
    humansand "weight teleportation" page, "Working with low-precision RL",
    pairs gate and up weights in groups of 64); the same tensor table, so
    the same plan fingerprint.
    """
    assert vocab % tp == 0 and ffn % tp == 0 and n_kv % tp == 0 and hidden % tp == 0
    assert gate_up_group == 0 or (ffn // tp) % gate_up_group == 0
    assert n_q * head_dim == hidden and n_q % n_kv == 0
    b = _Builder(name, seed)
    thr = rate_thr(rate)
    qpg = n_q // n_kv                       # q heads per kv group
    grp_rows = (qpg + 2) * head_dim         # rows of one [q.., k, v] group
    gpr = n_kv // tp                        # groups per rank
    kv = n_kv * head_dim
    v_r, f_r, h_r = vocab // tp, ffn // tp, hidden // tp
    recipe = []                             # (tensor id, how to assemble)

    def bf16_shard(n):
        s = b.shard(n, 2)
        b.region(s, 0, n, GEN_BF16, thr)
        return s

    def row_blocks(tname, rows, cols, per_rank_rows, shard_ids, route=ROUTE_AFFINE_XOR):
        t = b.tensor(tname, rows * cols, 2, route)
        for r, s in enumerate(shard_ids):
            b.seg(t, s, 0, r * per_rank_rows * cols, [per_rank_rows * cols], [1], [1])
        recipe.append((t, "cat0", [(s, 0, per_rank_rows, cols) for s in shard_ids]))
        return t

    emb = [bf16_shard(v_r * hidden) for _ in range(tp)]
    row_blocks("model.embed_tokens.weight", vocab, hidden, v_r, emb)
    for L in range(layers):
        p = f"model.layers.{L}."
        ln1 = bf16_shard(hidden)
        qkv = [bf16_shard(gpr * grp_rows * hidden) for _ in range(tp)]
        o = [bf16_shard(hidden * h_r) for _ in range(tp)]
        ln2 = bf16_shard(hidden)
        fc1 = [bf16_shard(2 * f_r * hidden) for _ in range(tp)]
        down = [bf16_shard(hidden * f_r) for _ in range(tp)]
        t = b.tensor(p + "input_layernorm.weight", hidden, 2)
        b.seg(t, ln1, 0, 0, [hidden], [1], [1])
        recipe.append((t, "whole", [ln1]))
        # fused QKV -> canonical q, k, v (residual path: overwrite records)
        tq = b.tensor(p + "self_attn.q_proj.weight", hidden * hidden, 2, ROUTE_OVERWRITE)
        tk = b.tensor(p + "self_attn.k_proj.weight", kv * hidden, 2, ROUTE_OVERWRITE)
        tv = b.tensor(p + "self_attn.v_proj.weight", kv * hidden, 2, ROUTE_OVERWRITE)
        pieces = {tq: [], tk: [], tv: []}
        for r in range(tp):
            for g in range(gpr):
                G = r * gpr + g
                base = g * grp_rows
                qr, kr = qpg * head_dim, head_dim
                b.seg(tq, qkv[r], base * hidden, G * qr * hidden, [qr * hidden], [1], [1])
                b.seg(tk, qkv[r], (base + qr) * hidden, G * kr * hidden, [kr * hidden], [1], [1])
                b.seg(tv, qkv[r], (base + qr + kr) * hidden, G * kr * hidden, [kr * hidden], [1], [1])
                pieces[tq].append((qkv[r], base, qr, hidden))
                pieces[tk].append((qkv[r], base + qr, kr, hidden))
                pieces[tv].append((qkv[r], base + qr + kr, kr, hidden))
        for t_ in (tq, tk, tv):
            recipe.append((t_, "cat0", pieces[t_]))
        # o_proj: row-parallel, rank r holds input columns [r*h_r, (r+1)*h_r)
        t = b.tensor(p + "self_attn.o_proj.weight", hidden * hidden, 2)
        for r in range(tp):
            b.seg(t, o[r], 0, r * h_r, [hidden, h_r], [h_r, 1], [hidden, 1])
        recipe.append((t, "cat1", [(s, hidden, h_r) for s in o]))
        t = b.tensor(p + "post_attention_layernorm.weight", hidden, 2)
        b.seg(t, ln2, 0, 0, [hidden], [1], [1])
        recipe.append((t, "whole", [ln2]))
        tg = b.tensor(p + "mlp.gate_proj.weight", ffn * hidden, 2)
        tu = b.tensor(p + "mlp.up_proj.weight", ffn * hidden, 2)
        if gate_up_group:
            gg = gate_up_group
            for r in range(tp):
                # row block j of g rows: gate at fused rows [2gj, 2gj + g), up at [2gj + g, 2g(j + 1))
                b.seg(tg, fc1[r], 0, r * f_r * hidden, [f_r // gg, gg * hidden], [2 * gg * hidden, 1],
                      [gg * hidden, 1])
                b.seg(tu, fc1[r], gg * hidden, r * f_r * hidden, [f_r // gg, gg * hidden], [2 * gg * hidden, 1],
                      [gg * hidden, 1])
            recipe.append((tg, "interleave", [(fc1[r], 0, gg, f_r, hidden) for r in range(tp)]))
            recipe.append((tu, "interleave", [(fc1[r], 1, gg, f_r, hidden) for r in range(tp)]))
        else:
            for r in range(tp):
                b.seg(tg, fc1[r], 0, r * f_r * hidden, [f_r * hidden], [1], [1])
                b.seg(tu, fc1[r], f_r * hidden, r * f_r * hidden, [f_r * hidden], [1], [1])
            recipe.append((tg, "cat0", [(fc1[r], 0, f_r, hidden) for r in range(tp)]))
            recipe.append((tu, "cat0", [(fc1[r], f_r, f_r, hidden) for r in range(tp)]))
        t = b.tensor(p + "mlp.down_proj.weight", hidden * ffn, 2)
        for r in range(tp):
            b.seg(t, down[r], 0, r * f_r, [hidden, f_r], [f_r, 1], [ffn, 1])
        recipe.append((t, "cat1", [(s, hidden, f_r) for s in down]))
    fn = bf16_shard(hidden)
    t = b.tensor("model.norm.weight", hidden, 2)
    b.seg(t, fn, 0, 0, [hidden], [1], [1])
    recipe.append((t, "whole", [fn]))
    head = [bf16_shard(v_r * hidden) for _ in range(tp)]
    row_blocks("lm_head.weight", vocab, hidden, v_r, head)

    def assemble(shards):
        return _assemble(recipe, shards, len(b.tensors))

    return b.build(assemble=assemble, meta={"seed": seed, "rate": rate, "tp": tp, "gate_up_group": gate_up_group})


def _assemble(recipe, shards, n_tensors):
    """Canonical tensors from shards using only library view / cat ops."""
    import torch
    out = [None] * n_tensors
    for t, how, parts in recipe:
        if how == "whole":
            out[t] = shards[parts[0]].reshape(-1)
        elif how == "cat0":        # row blocks: (shard, first row, rows, cols)
            out[t] = torch.cat([shards[s].reshape(-1, c).narrow(0, r0, nr)
                                for s, r0, nr, c in parts], 0).reshape(-1)
        elif how == "cat1":        # column blocks: (shard, rows, cols)
            out[t] = torch.cat([shards[s].reshape(rows, c) for s, rows, c in parts], 1).reshape(-1)
        elif how == "interleave":  # every other group of g rows: (shard, 0 or 1, g, rows, cols) per rank
            out[t] = torch.cat([shards[s].reshape(rows // g, 2, g, c).select(1, k).reshape(rows, c)
                                for s, k, g, rows, c in parts], 0).reshape(-1)
        elif how == "stack_sel":   # one matrix out of a stack: (shard, index, rows, cols)
            s, e, rows, c = parts
            out[t] = shards[s].reshape(-1, rows, c)[e].reshape(-1)
        else:
            raise ValueError(how)
    return out


# ------------------------------------------------------ random test layouts

CFG1_LR = float(np.uint32(901110982).view(np.float32))  # bisected once, see config1_values


def receiver_layout(lay: Layout, seed: int, n_shards_per_width=2) -> Layout:
    """Another physical layout of the same canonical tensors (same tensor
    table, hence the same plan fingerprint), as a receiver might store them.
    Each tensor is, at random: stored whole; cut at random (unaligned) points
    into contiguous pieces spread over the width's shards; cut into blocks of
    a random size stored in reverse order; or stored transposed as 2-D
    [rows, cols] for a random divisor cols of its size.  Every placement
    starts after a random gap of 0-9 elements, which no segment covers.  The
    layout carries no generated contents (regions)."""
    rng = np.random.default_rng(seed)
    b = _Builder(f"{lay.name}.recv{seed}", seed)
    for name, tt in zip(lay.tensor_names, lay.tensors):
        b.tensor(name, int(tt["numel"]), int(tt["elem_bytes"]), int(tt["route"]), int(tt["scale_tensor"]),
                 int(tt["scale_block"]))
    shards = {}      # width -> shard ids
    fill = []        # elements used per shard

    def shard_of(w):
        if w not in shards:
            shards[w] = []
            for _ in range(n_shards_per_width):
                shards[w].append(b.shard(0, w))
                fill.append(0)
        return shards[w][int(rng.integers(0, len(shards[w])))]

    def place(s, n):
        off = fill[s] + int(rng.integers(0, 10))
        fill[s] = off + n
        return off

    for t, tt in enumerate(lay.tensors):
        n, w = int(tt["numel"]), int(tt["elem_bytes"])
        if n == 0:
            continue
        divs = [d for d in (3, 5, 7, 8, 24, 100, 129, 256, 1000, 4096) if n % d == 0 and 1 < d < n]
        how = rng.choice(["whole", "pieces", "blocks", "transpose"] if divs else ["whole", "pieces", "blocks"])
        if how == "whole":
            s = shard_of(w)
            b.seg(t, s, place(s, n), 0, [n], [1], [1])
        elif how == "pieces":
            k = int(rng.integers(2, 6))
            cuts = sorted(set(int(x) for x in rng.integers(1, n, size=k - 1))) if n > 1 else []
            bounds = [0] + cuts + [n]
            for i in range(len(bounds) - 1):
                e0, e1 = bounds[i], bounds[i + 1]
                s = shard_of(w)
                b.seg(t, s, place(s, e1 - e0), e0, [e1 - e0], [1], [1])
        elif how == "blocks":
            blk = int(rng.integers(1, 5000))
            s = shard_of(w)
            starts = list(range(0, n, blk))[::-1]
            for e0 in starts:
                e1 = min(n, e0 + blk)
                b.seg(t, s, place(s, e1 - e0), e0, [e1 - e0], [1], [1])
        else:
            cols = int(rng.choice(divs))
            rows = n // cols
            s = shard_of(w)
            b.seg(t, s, place(s, n), 0, [rows, cols], [1, rows], [cols, 1])
    for s in range(len(fill)):
        b.shard_elems[s] = fill[s] + int(rng.integers(0, 10))
    return b.build(meta={"seed": seed, "receiver_of": lay.name})


def scatter_canonical_gpu(lay: Layout, canon, device="cuda", fill=0xA5):
    """Device shards of layout `lay` holding the canonical tensors `canon`
    (numpy arrays or device tensors, any element view): every segment is
    copied with strided views; bytes no segment covers hold `fill`.
    Returns (buffer, per-shard byte views)."""
    import torch
    buf, shards = alloc_shards(lay, device)
    buf.fill_(fill)
    dts = {1: torch.uint8, 2: torch.int16, 4: torch.int32}
    cdev = [c if isinstance(c, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(c)).to(device)
            for c in canon]
    for g in lay.segments:
        t, s, nd = int(g["tensor_id"]), int(g["shard_id"]), int(g["ndim"])
        dt = dts[int(lay.tensors[t]["elem_bytes"])]
        sv = shards[s].view(dt)
        cv = cdev[t].reshape(-1).view(torch.uint8).view(dt)
        size = [int(x) for x in g["extent"][:nd]]
        dst = sv.as_strided(size, [int(x) for x in g["shard_stride"][:nd]], sv.storage_offset() + int(g["shard_off"]))
        src = cv.as_strided(size, [int(x) for x in g["canon_stride"][:nd]], cv.storage_offset() + int(g["canon_off"]))
        dst.copy_(src)
    return buf, shards


def random_layout(seed: int, max_tensors=4, max_chunks=3.0, allow_transpose=True,
                  allow_block_scaled=True, rate=None, widths=None) -> Layout:
    """A small random layout with explicit random contents, for property tests.

    Tensors are 2-D [rows, cols] with 1- or 2-byte elements (plus fp32 scale
    tensors for block-scaled ones) and odd sizes; each is stored whole, split
    into uneven row blocks or uneven column blocks over several shards, or
    stored transposed; several tensors may share a shard.  Old contents are
    uniform random bits; a random fraction of elements gets random new bits
    (sign flips, low-bit and high-bit changes).  widths: element widths
    given to the tensors in turn (at least one tensor each) instead of the
    random choice; a 4-byte tensor is an overwrite tensor of its own.
    """
    rng = np.random.default_rng(seed)
    b = _Builder(f"rand{seed}", seed)
    recipes = []
    shard_parts = []   # per shard: list of numpy arrays to concatenate (with padding)
    rate = rate if rate is not None else float(rng.choice([0.002, 0.03, 0.2, 0.7]))

    def new_shard(n, w):
        s = b.shard(0, w)
        shard_parts.append([])
        return s

    def place(s, n, w):
        """Reserve n elements in shard s (after random padding); return offset."""
        pad = int(rng.integers(0, 9))
        off = sum(len(a) for a in shard_parts[s]) + pad
        dt = {1: np.uint8, 2: np.uint16, 4: np.uint32}[w]
        shard_parts[s].append(np.zeros(pad, dtype=dt))
        shard_parts[s].append(np.zeros(n, dtype=dt))
        return off, len(shard_parts[s]) - 1

    n_t = int(rng.integers(1, max_tensors + 1))
    if widths is not None:
        n_t = max(n_t, len(widths))
    canon_vals = []
    pending_fill = []
    shared = {}
    for ti in range(n_t):
        w = int(rng.choice([1, 2, 2, 2])) if widths is None else int(widths[ti % len(widths)])
        E = 65536 // w
        numel_target = int(rng.integers(0, int(max_chunks * E) + 2))
        cols = int(rng.choice([1, 3, 8, 24, 100, 129, 256, 1000, 4096]))
        rows = max(numel_target // cols, 0) if numel_target else 0
        if rng.random() < 0.1:
            rows = 0
        numel = rows * cols
        route = int(rng.choice([ROUTE_AFFINE_XOR, ROUTE_AFFINE_XOR, ROUTE_OVERWRITE,
                                ROUTE_BLOCK_SCALED if allow_block_scaled else ROUTE_AFFINE_XOR]))
        if w == 4:
            route = ROUTE_OVERWRITE
        sb = 0
        if route == ROUTE_BLOCK_SCALED:
            sb = int(rng.choice([16, 32, 128, 256])) if w == 1 else int(rng.choice([8, 64, 128]))
        t = b.tensor(f"t{ti}", numel, w, route, -1, sb)
        mode = rng.choice(["whole", "rows", "cols", "transpose"] if allow_transpose and numel <= 40000
                          else ["whole", "rows", "cols"])
        if numel == 0:
            mode = "whole"
        dt = {1: np.uint8, 2: np.uint16, 4: np.uint32}[w]
        old = rng.integers(0, 1 << (8 * w), size=numel, dtype=np.uint64).astype(dt)
        canon_vals.append((t, rows, cols, w, old))
        if mode == "whole":
            key = ("shared", w)
            s = shared.get(key)
            if s is None or rng.random() < 0.5:
                s = new_shard(0, w)
                shared[key] = s
            off, part = place(s, numel, w)
            b.seg(t, s, off, 0, [numel], [1], [1])
            pending_fill.append((s, part, lambda c, rows=rows, cols=cols: c.reshape(-1)))
            recipes.append((t, "whole", [(s, off, numel)]))
        elif mode == "rows":
            k = int(rng.integers(1, 5))
            cuts = sorted(rng.integers(0, rows + 1, size=k - 1).tolist()) if rows else []
            bounds = [0] + cuts + [rows]
            parts = []
            for i in range(k):
                r0, r1 = bounds[i], bounds[i + 1]
                s = new_shard(0, w)
                off, part = place(s, (r1 - r0) * cols, w)
                if r1 > r0:
                    b.seg(t, s, off, r0 * cols, [(r1 - r0) * cols], [1], [1])
                pending_fill.append((s, part, lambda c, r0=r0, r1=r1, cols=cols:
                                     c.reshape(-1, cols)[r0:r1].reshape(-1)))
                parts.append((s, off, r1 - r0, cols))
            recipes.append((t, "rows", parts))
        elif mode == "cols":
            k = int(rng.integers(1, 5))
            cuts = sorted(rng.integers(0, cols + 1, size=k - 1).tolist())
            bounds = [0] + cuts + [cols]
            parts = []
            for i in range(k):
                c0, c1 = bounds[i], bounds[i + 1]
                s = new_shard(0, w)
                off, part = place(s, rows * (c1 - c0), w)
                if c1 > c0 and rows:
                    b.seg(t, s, off, c0, [rows, c1 - c0], [c1 - c0, 1], [cols, 1])
                pending_fill.append((s, part, lambda c, c0=c0, c1=c1, cols=cols:
                                     c.reshape(-1, cols)[:, c0:c1].reshape(-1)))
                parts.append((s, off, rows, c1 - c0))
            recipes.append((t, "cols", parts))
        else:  # transpose: shard holds [cols, rows]
            s = new_shard(0, w)
            off, part = place(s, numel, w)
            b.seg(t, s, off, 0, [rows, cols], [1, rows], [cols, 1])
            pending_fill.append((s, part, lambda c, cols=cols: c.reshape(-1, cols).T.reshape(-1)))
            recipes.append((t, "transpose", [(s, off, rows, cols)]))
        if route == ROUTE_BLOCK_SCALED:
            ns = (numel + sb - 1) // sb
            st = b.tensor(f"t{ti}.scale", ns, 4, ROUTE_OVERWRITE)
            b.tensors[t] = (numel, w, route, st, sb)
            s = new_shard(0, 4)
            off, part = place(s, ns, 4)
            b.seg(st, s, off, 0, [ns], [1], [1])
            sold = rng.integers(0, 1 << 32, size=ns, dtype=np.uint64).astype(np.uint32)
            canon_vals.append((st, ns, 1, 4, sold))
            pending_fill.append((s, part, lambda c: c.reshape(-1)))
            recipes.append((st, "whole", [(s, off, ns)]))
            # pending_fill entries are matched to canon_vals by tensor order below
    # new canonical values: random bit changes
    canon_new = []
    for (t, rows, cols, w, old) in canon_vals:
        n = old.size
        ch = rng.random(n) < rate
        kindsel = rng.integers(0, 4, size=n)
        bits = 8 * w
        rnd = rng.integers(1, 1 << bits, size=n, dtype=np.uint64)
        low = rng.integers(1, 256, size=n, dtype=np.uint64)
        sign = np.uint64(1 << (bits - 1))
        mask = np.where(kindsel == 0, sign, np.where(kindsel == 1, low, rnd)).astype(old.dtype)
        new = np.where(ch, old ^ mask, old).astype(old.dtype)
        canon_new.append(new)
    # fill shard parts from canonical old/new via the recipe lambdas
    old_parts = [[a.copy() for a in parts] for parts in shard_parts]
    new_parts = [[a.copy() for a in parts] for parts in shard_parts]
    fills = iter(pending_fill)
    for (t, rows, cols, w, old), new in zip(canon_vals, canon_new):
        nparts = recipe_nparts(recipes, t)
        for _ in range(nparts):
            s, part, fn = next(fills)
            old_parts[s][part][:] = fn(old)
            new_parts[s][part][:] = fn(new)
    olds = [np.concatenate(p) if p else np.zeros(0, dtype=np.uint8) for p in old_parts]
    news = [np.concatenate(p) if p else np.zeros(0, dtype=np.uint8) for p in new_parts]
    for s in range(len(olds)):
        b.shard_elems[s] = int(olds[s].size)
        if olds[s].size == 0:
            dt = {1: np.uint8, 2: np.uint16, 4: np.uint32}[b.shard_w[s]]
            olds[s] = np.zeros(0, dtype=dt)
            news[s] = np.zeros(0, dtype=dt)

    canon_old = {t: old for (t, _r, _c, _w, old) in canon_vals}
    canon_new_d = {t: new for (t, _r, _c, _w, _o), new in zip(canon_vals, canon_new)}

    def assemble(shards):
        return _assemble_random(recipes, shards, len(b.tensors))

    lay = b.build(assemble=assemble, meta={"seed": seed, "rate": rate,
                                           "canon_old": canon_old, "canon_new": canon_new_d})
    lay.values = (olds, news)
    return lay


def width_set_layout(ws: int, k: int = 0, rate=None) -> Layout:
    """A random layout whose non-empty tensors hold exactly the element
    widths of the bit set ws (1-, 2- and 4-byte elements; a 4-byte tensor
    also on its own, stored whole, split or transposed): the k-th such
    layout of the widths option from seed 2300 on (change rate as given,
    else the layout's own)."""
    widths = [w for w in (1, 2, 4) if ws & w]
    found = 0
    for seed in range(2300, 3300):
        lay = random_layout(seed, widths=widths, allow_block_scaled=bool(ws & 4), rate=rate)
        got = 0
        for t in lay.tensors:
            if int(t["numel"]):
                got |= int(t["elem_bytes"])
        if got == ws:
            if found == k:
                return lay
            found += 1
    raise ValueError(f"no layout of width set {ws}")


def recipes_kind(recipes, t):
    for tt, how, _ in recipes:
        if tt == t:
            return how
    raise KeyError(t)


def recipe_nparts(recipes, t):
    for tt, _how, parts in recipes:
        if tt == t:
            return len(parts)
    raise KeyError(t)


def _assemble_random(recipes, shards, n_tensors):
    """Canonical tensors from shards with library ops (works for numpy or torch)."""
    def cat(xs, axis):
        try:
            import torch
            if isinstance(xs[0], torch.Tensor):
                return torch.cat(xs, axis)
        except ImportError:
            pass
        return np.concatenate(xs, axis)

    out = [None] * n_tensors
    for t, how, parts in recipes:
        if how == "whole":
            s, off, n = parts[0]
            out[t] = shards[s][off:off + n]
        elif how == "rows":
            out[t] = cat([shards[s][off:off + nr * c].reshape(nr, c) for s, off, nr, c in parts], 0).reshape(-1)
        elif how == "cols":
            out[t] = cat([shards[s][off:off + r * nc].reshape(r, nc) for s, off, r, nc in parts], 1).reshape(-1)
        elif how == "transpose":
            s, off, rows, cols = parts[0]
            out[t] = shards[s][off:off + rows * cols].reshape(cols, rows).T.reshape(-1)
        else:
            raise ValueError(how)
    return out


# ---------------------------------------------------------- GPU generation

_synth_lib = None


def _load_synth():
    """libdcr_synth.so: the same generator definition on the GPU (untimed input setup)."""
    global _synth_lib
    if _synth_lib is None:
        import ctypes
        import os
        p = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdcr_synth.so")
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is missing: build it with `python -m bit_exact_xor_amd.build`")
        lib = ctypes.CDLL(p)
        U64, U32, P = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p
        lib.dcr_synth_fill.restype = ctypes.c_int32
        lib.dcr_synth_fill.argtypes = [P, U64, U64, U32, U64, U64, U64, U64, P, U64, U32, U64, U64, U32,
                                       U32, U32, P]
        lib.dcr_synth_read_probe.restype = ctypes.c_int32
        lib.dcr_synth_read_probe.argtypes = [P, U64, P, P]
        lib.dcr_synth_rmw_probe.restype = ctypes.c_int32
        lib.dcr_synth_rmw_probe.argtypes = [P, U64, P, P]
        lib.dcr_synth_rmw_lines_probe.restype = ctypes.c_int32
        lib.dcr_synth_rmw_lines_probe.argtypes = [P, U64, P, P]
        _synth_lib = lib
    return _synth_lib


def alloc_shards(lay: Layout, device="cuda", align=256):
    """One device buffer per version holding every shard at an aligned offset."""
    import torch
    offs, total = [], 0
    for s in range(lay.n_shards):
        offs.append(total)
        total += (lay.shard_bytes(s) + align - 1) // align * align
    buf = torch.empty(max(total, align), dtype=torch.uint8, device=device)
    return buf, [buf[o:o + lay.shard_bytes(s)] for s, o in enumerate(offs)]


def fill_shards_gpu(lay: Layout, shards, version: int, stream=None):
    """Generate every region of the layout into device shards (version 0 / 1)."""
    import torch
    lib = _load_synth()
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    hot_lists = [r.hot_rows for r in lay.regions if r.hot_rows is not None and len(r.hot_rows)]
    hot_dev = None
    if hot_lists:
        hot_dev = torch.from_numpy(np.concatenate(hot_lists).astype(np.uint32).view(np.int32)).to(shards[0].device)
    hot_off = 0
    for r in lay.regions:
        n_hot = 0 if r.hot_rows is None else len(r.hot_rows)
        rc = lib.dcr_synth_fill(shards[r.shard].data_ptr(), r.elem_off, r.n, r.kind, r.key_old, r.key_chg,
                                r.thr, r.row_len, hot_dev.data_ptr() if n_hot else None, hot_off, n_hot,
                                r.key_blk, r.thr_blk, r.blk, version, SCALE_BITS, stream or None)
        if rc:
            raise RuntimeError(f"dcr_synth_fill failed: {rc}")
        hot_off += n_hot
    return hot_dev  # keep alive until the fills have run


def read_probe_gpu(buf, sink, stream=None):
    """One streaming read of the device tensor `buf` (bandwidth probe)."""
    import torch
    lib = _load_synth()
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    n = buf.numel() * buf.element_size() // 16 * 16
    rc = lib.dcr_synth_read_probe(buf.data_ptr(), n, sink.data_ptr(), stream or None)
    if rc:
        raise RuntimeError(f"dcr_synth_read_probe failed: {rc}")
    return n


def rmw_probe_gpu(buf, bits, stream=None, whole_lines=False):
    """XOR a fixed mask into the 16-byte groups of the device tensor `buf`
    whose bits are set in the device bit array `bits` (LSB first, one bit per
    group; bandwidth probe for the in-place patch pattern).  whole_lines:
    every 128-byte line holding a set group (eight groups from the buffer's
    start) is read and written whole, the other groups unchanged."""
    import torch
    lib = _load_synth()
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    n = buf.numel() * buf.element_size()
    groups = n // 16
    if n % 16 or bits.numel() * bits.element_size() < (groups + 15) // 16 * 2:
        raise ValueError("rmw_probe_gpu: buffer not a multiple of 16 bytes, or too few bits")
    fn = lib.dcr_synth_rmw_lines_probe if whole_lines else lib.dcr_synth_rmw_probe
    rc = fn(buf.data_ptr(), n, bits.data_ptr(), stream or None)
    if rc:
        raise RuntimeError(f"rmw probe failed: {rc}")


# ------------------------------------------------- configs 3 / 4 (MoE)

def _uniforms(key: int, n: int) -> np.ndarray:
    return (hashes(key, 0, n) >> np.uint64(11)).astype(np.float64) / float(1 << 53)


def beta_2_60_rates(seed: int, numels: np.ndarray, mean: float) -> np.ndarray:
    """One Beta(2, 60) draw per tensor (the 2nd smallest of 61 uniforms), then
    rescaled so that the numel-weighted mean is `mean`; clamped to [0, 1]."""
    n = len(numels)
    u = _uniforms(derive_key(seed, 7777, 0), 61 * n).reshape(n, 61)
    r = np.sort(u, axis=1)[:, 1]
    w = numels.astype(np.float64)
    r = r * mean * w.sum() / (r * w).sum()
    return np.minimum(r, 1.0)


def _hot_rows(seed: int, stream: int, rows: int, frac: float) -> np.ndarray:
    """frac of the rows (at least one): the first ranks of a seeded permutation
    of the row ids (the most-hit ids under a Zipf(1.1) popularity law)."""
    k = max(1, int(np.ceil(frac * rows)))
    order = np.argsort(hashes(derive_key(seed, 9000 + stream, 0), 0, rows), kind="stable")
    return np.sort(order[:k]).astype(np.uint32)


def moe_layout(hidden=2048, layers=48, n_exp=128, moe_ffn=768, n_q=32, n_kv=4, head_dim=128,
               vocab=151936, ep=8, rate=0.03, variant="beta", seed=0xDC202603, name="cfg3",
               hot_frac=0.01, scale_block=128, ow_share=0.05) -> Layout:
    """Qwen3-30B-A3B-shaped MoE checkpoint, experts sharded EP=ep.

    Trainer shards: each rank holds its n_exp/ep experts of every layer as
    stacked tensors gate [E_r, moe_ffn, hidden], up [E_r, moe_ffn, hidden],
    down [E_r, hidden, moe_ffn]; every non-expert tensor is stored whole and
    owned by rank 0 (identity projection).  Canonical tensors are per expert.

    variant "beta": per canonical tensor a change rate drawn from Beta(2,60),
    rescaled to a `rate` (numel-weighted) mean; +-1 ulp changes.
    variant "hot": `rate` overall with hot rows (hot_frac of the rows of
    every 2-D tensor change at 100 %) and block-scaled experts: each expert
    tensor gets an fp32 scale tensor of one scale per `scale_block` elements;
    a changed scale changes its whole block (OW route), for `ow_share` of all
    changes; the remaining changes are uniform.
    """
    assert n_exp % ep == 0 and n_q * head_dim >= hidden // 2
    b = _Builder(name, seed)
    e_r = n_exp // ep
    q_out, kv_out = n_q * head_dim, n_kv * head_dim
    hot = variant == "hot"
    recipe = []
    # ---- canonical tensors (id order = record order)
    specs = []   # (name, rows, cols, kind, extra)
    specs.append(("model.embed_tokens.weight", vocab, hidden, "whole", None))
    for L in range(layers):
        p = f"model.layers.{L}."
        specs += [(p + "input_layernorm.weight", 1, hidden, "whole", None),
                  (p + "self_attn.q_proj.weight", q_out, hidden, "whole", None),
                  (p + "self_attn.k_proj.weight", kv_out, hidden, "whole", None),
                  (p + "self_attn.v_proj.weight", kv_out, hidden, "whole", None),
                  (p + "self_attn.o_proj.weight", hidden, q_out, "whole", None),
                  (p + "self_attn.q_norm.weight", 1, head_dim, "whole", None),
                  (p + "self_attn.k_norm.weight", 1, head_dim, "whole", None),
                  (p + "post_attention_layernorm.weight", 1, hidden, "whole", None),
                  (p + "mlp.gate.weight", n_exp, hidden, "whole", None)]
        for e in range(n_exp):
            for proj, rows, cols in (("gate_proj", moe_ffn, hidden), ("up_proj", moe_ffn, hidden),
                                     ("down_proj", hidden, moe_ffn)):
                specs.append((p + f"mlp.experts.{e}.{proj}.weight", rows, cols, "expert", (L, e, proj)))
    specs.append(("model.norm.weight", 1, hidden, "whole", None))
    specs.append(("lm_head.weight", vocab, hidden, "whole", None))
    numels = np.array([r * c for _, r, c, _, _ in specs], dtype=np.int64)

    if hot:
        expert_numel = sum(n for (_, _, _, k, _), n in zip(specs, numels) if k == "expert")
        total = numels.sum()
        p_blk = ow_share * rate * total / expert_numel            # scale-block hit probability
        hot_elems = sum(n * hot_frac for (_, r, _, _, _), n in zip(specs, numels) if r > 1)
        base = (rate * total - hot_elems - p_blk * expert_numel) / (total - hot_elems - p_blk * expert_numel)
        rates = np.full(len(specs), max(base, 0.0))
        thr_blk = rate_thr(p_blk)
    else:
        rates = beta_2_60_rates(seed, numels, rate)
        thr_blk = 0

    # ---- shards: stacked expert shards per (layer, rank, proj); others whole
    tid = {}
    stack_shard = {}
    scale_stack = {}
    for i, (nm, rows, cols, kind, extra) in enumerate(specs):
        route = ROUTE_BLOCK_SCALED if (hot and kind == "expert") else ROUTE_AFFINE_XOR
        t = b.tensor(nm, rows * cols, 2, route, -1, 0)
        tid[nm] = t
        if hot and kind == "expert":
            ns = (rows * cols + scale_block - 1) // scale_block
            st = b.tensor(nm + "_scale", ns, 4, ROUTE_OVERWRITE)
            b.tensors[t] = (rows * cols, 2, route, st, scale_block)
        if kind == "whole":
            s = b.shard(rows * cols, 2)
            b.seg(t, s, 0, 0, [rows * cols], [1], [1])
            hr = _hot_rows(seed, t, rows, hot_frac) if (hot and rows > 1) else None
            b.region(s, 0, rows * cols, GEN_BF16_HOT if hot else GEN_BF16, rate_thr(rates[i]),
                     row_len=cols, hot_rows=hr)
            recipe.append((t, "whole", [s]))
        else:
            L, e, proj = extra
            r_ = e // e_r
            j = e % e_r
            key = (L, r_, proj)
            if key not in stack_shard:
                stack_shard[key] = b.shard(e_r * rows * cols, 2)
                if hot:
                    scale_stack[key] = b.shard(e_r * ((rows * cols + scale_block - 1) // scale_block), 4)
            s = stack_shard[key]
            b.seg(t, s, j * rows * cols, 0, [rows * cols], [1], [1])
            recipe.append((t, "stack_sel", (s, j, rows, cols)))
            if hot:
                ns = (rows * cols + scale_block - 1) // scale_block
                kblk = derive_key(seed, 50000 + t, 1)
                hr = _hot_rows(seed, t, rows, hot_frac)
                b.region(s, j * rows * cols, rows * cols, GEN_BF16_HOT, rate_thr(rates[i]), row_len=cols,
                         hot_rows=hr, key_blk=kblk, thr_blk=thr_blk, blk=scale_block)
                ss = scale_stack[key]
                st = b.tensors[t][3]
                b.seg(st, ss, j * ns, 0, [ns], [1], [1])
                b.region(ss, j * ns, ns, GEN_F32SCALE, thr_blk, key_chg=kblk)
                recipe.append((st, "stack_sel", (ss, j, 1, ns)))
            else:
                b.region(s, j * rows * cols, rows * cols, GEN_BF16, rate_thr(rates[i]))

    def assemble(shards):
        return _assemble(recipe, shards, len(b.tensors))

    return b.build(assemble=assemble, meta={"seed": seed, "rate": rate, "variant": variant, "ep": ep,
                                            "rates": rates})


def config3_layout(**kw) -> Layout:
    return moe_layout(rate=0.03, variant="beta", seed=0xDC202603, name="cfg3", **kw)


def config4_layout(**kw) -> Layout:
    return moe_layout(rate=0.05, variant="hot", seed=0xDC202604, name="cfg4", **kw)


def sub_layout(lay: Layout, tensor_ids):
    """The inputs of a subset of tensors as a small layout of their own: each
    segment reads a private mini-shard holding just the shard range it
    touches, generated on the CPU from the same regions.  Returns
    (tensors, segments, old mini-shards, new mini-shards); tensor ids are
    renumbered in the given order (scale links follow when both are kept)."""
    tensor_ids = list(tensor_ids)
    remap = {t: i for i, t in enumerate(tensor_ids)}
    T = lay.tensors[tensor_ids].copy()
    for i, t in enumerate(tensor_ids):
        st = int(lay.tensors[t]["scale_tensor"])
        if st >= 0:
            assert st in remap, "keep a block-scaled tensor's scale tensor in the subset"
            T[i]["scale_tensor"] = remap[st]
    segs, olds, news = [], [], []
    for g in lay.segments:
        t = int(g["tensor_id"])
        if t not in remap:
            continue
        nd = int(g["ndim"])
        ext = [int(x) for x in g["extent"][:nd]]
        ss = [int(x) for x in g["shard_stride"][:nd]]
        lo = int(g["shard_off"]) + sum(min(0, (e - 1) * s) for e, s in zip(ext, ss))
        hi = int(g["shard_off"]) + sum(max(0, (e - 1) * s) for e, s in zip(ext, ss)) + 1
        s = int(g["shard_id"])
        w = lay.shard_w[s]
        dt = {1: np.uint8, 2: np.uint16, 4: np.uint32}[w]
        mo, mn = np.zeros(hi - lo, dtype=dt), np.zeros(hi - lo, dtype=dt)
        for r in lay.regions:
            if r.shard != s:
                continue
            a, b_ = max(lo, r.elem_off), min(hi, r.elem_off + r.n)
            if a >= b_:
                continue
            for v, out in ((0, mo), (1, mn)):
                out[a - lo:b_ - lo] = gen_region(r.kind, r.key_old, r.key_chg, r.thr, a - r.elem_off, b_ - a,
                                                 v, r.row_len, r.hot_rows, r.key_blk, r.thr_blk, r.blk)
        g2 = g.copy()
        g2["tensor_id"] = remap[t]
        g2["shard_id"] = len(olds)
        g2["shard_off"] = int(g["shard_off"]) - lo
        segs.append(g2)
        olds.append(mo)
        news.append(mn)
    S = np.array(segs, dtype=SEGMENT_DT) if segs else np.zeros(0, dtype=SEGMENT_DT)
    return T, S, olds, news


# ------------------------------------------------ config 5 (receiver share)

def config5_layout(n_bf16=6812, bf16_shape=(7168, 2048), n_u8=5450, u8_shape=(7168, 1024),
                   rate_bf16=0.03, rate_u8=0.00085, seed=0xDC202605) -> Layout:
    """One GPU's receiver share of a 1T-parameter model: n_bf16 BF16 tensors
    (100 B parameters, 200 GB) and n_u8 uint8 NVFP4-packed tensors (40 GB),
    each stored whole (identity projection, shard i = tensor i)."""
    b = _Builder("cfg5", seed)
    recipe = []
    for i in range(n_bf16):
        n = bf16_shape[0] * bf16_shape[1]
        t = b.tensor(f"bf16.{i}", n, 2)
        s = b.shard(n, 2)
        b.seg(t, s, 0, 0, [n], [1], [1])
        b.region(s, 0, n, GEN_BF16, rate_thr(rate_bf16))
        recipe.append((t, "whole", [s]))
    for i in range(n_u8):
        n = u8_shape[0] * u8_shape[1]
        t = b.tensor(f"nvfp4.{i}", n, 1)
        s = b.shard(n, 1)
        b.seg(t, s, 0, 0, [n], [1], [1])
        b.region(s, 0, n, GEN_U8, rate_thr(rate_u8))
        recipe.append((t, "whole", [s]))

    def assemble(shards):
        return _assemble(recipe, shards, len(b.tensors))

    return b.build(assemble=assemble, meta={"seed": seed})


def window_layout(lay: Layout, a: int, b_: int) -> Layout:
    """Tensors [a, b_) of an identity layout (shard i = tensor i) as a layout of
    their own, with shard and tensor ids renumbered from 0."""
    T = lay.tensors[a:b_].copy()
    S = lay.segments[a:b_].copy()
    S["tensor_id"] = np.arange(b_ - a)
    S["shard_id"] = np.arange(b_ - a)
    regions = []
    for r in lay.regions[a:b_]:
        regions.append(dataclasses.replace(r, shard=r.shard - a))
    return Layout(f"{lay.name}[{a}:{b_}]", lay.tensor_names[a:b_], T, S, lay.shard_elems[a:b_],
                  lay.shard_w[a:b_], regions, None, {})
