"""ctypes wrapper of the CPU oracle (``liboracle.so``) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The product path never does.

The oracle is the plain single-threaded definition of bit-exact delta refit
(bit-pattern change detection, direct projection to canonical coordinates,
XOR / overwrite records, in-place apply with dedup flags, overwrite retry),
written from the NeMo-DCR pages (ai-feeds summary "Method"; tokendh blog
"shard owner", "XOR or overwrite", "no backup copy"; ai.info abstract) and the
delta algebra of the humansand "weight teleportation" page.  See
``dcr_oracle.h`` for the per-function citations.

Inputs are numpy arrays; the tensor table and the segment list are given as
numpy structured arrays (or anything with the same field names) and are
packed here into the oracle's own C structs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SOURCES = [os.path.join(_HERE, "dcr_oracle.c")]

OK, E_INVAL, E_COVERAGE, E_FORMAT, E_VERSION, E_CAPACITY, E_NOMEM = 0, -1, -2, -3, -4, -5, -7
ROUTE_AFFINE_XOR, ROUTE_OVERWRITE, ROUTE_BLOCK_SCALED = 0, 1, 2
MODE_DELTA, MODE_RETRY = 0, 1
ENC_LISTS = 0x100                 # encode option: index-list layout for low-density records
LAYOUT_BITMAP, LAYOUT_LIST = 0, 1
KIND_XOR, KIND_OW = 0, 1
HI_NONE, HI_SPARSE, HI_DENSE = 0, 1, 2
HEADER_BYTES, DIRENT_BYTES, CHUNK_BYTES = 64, 32, 65536

# The oracle's own binary layouts of its input structs.
ORC_TENSOR = np.dtype([("numel", "<u8"), ("elem_bytes", "<u4"), ("route", "<u4"),
                       ("scale_tensor", "<i4"), ("scale_block", "<u4")])
ORC_SEGMENT = np.dtype([("tensor_id", "<u4"), ("shard_id", "<u4"), ("ndim", "<u4"),
                        ("reserved", "<u4"), ("shard_off", "<u8"), ("canon_off", "<u8"),
                        ("extent", "<u8", (4,)), ("shard_stride", "<i8", (4,)),
                        ("canon_stride", "<i8", (4,))])
assert ORC_TENSOR.itemsize == 24 and ORC_SEGMENT.itemsize == 128


def build(force: bool = False, extra_flags: tuple = (), src_dir: str | None = None,
          out_path: str | None = None) -> str:
    """Compile the oracle with gcc (plain C99, -O2, one thread)."""
    out = out_path or LIB_PATH
    srcs = SOURCES if src_dir is None else [os.path.join(src_dir, "dcr_oracle.c")]
    if not force and os.path.exists(out) and all(
            os.path.getmtime(out) >= os.path.getmtime(s) for s in srcs):
        return out
    inc = os.path.dirname(srcs[0])
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-fPIC", "-shared",
           "-I", inc, *extra_flags, "-o", out + ".tmp", *srcs]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _pack(arr, dtype):
    out = np.zeros(len(arr), dtype=dtype)
    for name in dtype.names:
        if name == "reserved":
            continue
        out[name] = arr[name]
    return out


class Oracle:
    """One loaded oracle library (a mutated copy can be loaded from another path)."""

    def __init__(self, path: str | None = None):
        self.path = path or build()
        lib = ctypes.CDLL(self.path)
        P, U32, U64, I32 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int32
        U64P = ctypes.POINTER(ctypes.c_uint64)
        lib.orc_fingerprint.restype = U64
        lib.orc_fingerprint.argtypes = [P, U32]
        lib.orc_encode.restype = I32
        lib.orc_encode.argtypes = [P, U32, P, P, P, U32, P, U64, U32, U64, U64,
                                   P, P, U64, U64P, P, U64, U64P]
        lib.orc_encode_retry_partial.restype = I32
        lib.orc_encode_retry_partial.argtypes = [P, U32, P, P, P, U32, P, U64, P, P, P, U64, U64,
                                                 P, P, U64, U64P, P, U64, U64P]
        lib.orc_gather.restype = I32
        lib.orc_gather.argtypes = [P, U32, P, P, U32, P, U64, U32, P]
        lib.orc_validate.restype = I32
        lib.orc_validate.argtypes = [P, U32, P, P, P, U64, I32]
        lib.orc_apply.restype = I32
        lib.orc_apply.argtypes = [P, U32, P, P, P, P, P, U64, U64, U64]
        lib.orc_apply_overwrite_retry.restype = I32
        lib.orc_apply_overwrite_retry.argtypes = [P, U32, P, P, P, P, U64]
        lib.orc_apply_record_part.restype = I32
        lib.orc_apply_record_part.argtypes = [P, U32, P, P, P, U64, U32, U32]
        for fn in (lib.orc_stream_pack, lib.orc_stream_unpack):
            fn.restype = I32
            fn.argtypes = [P, U32, P, P, P, P, P, P, U64, U64P]
        self.lib = lib

    # -------------------------------------------------------------- helpers
    @staticmethod
    def _ptrs(bufs):
        arr = (ctypes.c_void_p * max(1, len(bufs)))()
        for i, b in enumerate(bufs):
            arr[i] = b.ctypes.data if b.size else None
        return arr

    def fingerprint(self, tensors) -> int:
        T = _pack(tensors, ORC_TENSOR)
        return int(self.lib.orc_fingerprint(T.ctypes.data, len(T)))

    def gather(self, tensors, segments, shards, t: int) -> np.ndarray:
        T = _pack(tensors, ORC_TENSOR)
        S = _pack(segments, ORC_SEGMENT)
        shards = [np.ascontiguousarray(s).view(np.uint8).reshape(-1) for s in shards]
        sb = np.array([s.nbytes for s in shards], dtype=np.uint64)
        out = np.zeros(int(T[t]["numel"]) * int(T[t]["elem_bytes"]), dtype=np.uint8)
        rc = self.lib.orc_gather(T.ctypes.data, len(T), self._ptrs(shards), sb.ctypes.data,
                                 len(shards), S.ctypes.data, len(S), t, out.ctypes.data)
        if rc:
            raise OracleError(rc)
        return out

    def encode(self, tensors, segments, old_shards, new_shards, mode=MODE_DELTA,
               base_version=0, new_version=1, dir_cap=None, payload_cap=None):
        """Return (rc, header bytes, directory bytes, payload bytes)."""
        T = _pack(tensors, ORC_TENSOR)
        S = _pack(segments, ORC_SEGMENT)
        olds = [np.ascontiguousarray(s).view(np.uint8).reshape(-1) for s in old_shards]
        news = [np.ascontiguousarray(s).view(np.uint8).reshape(-1) for s in new_shards]
        sb = np.array([s.nbytes for s in olds], dtype=np.uint64)
        assert all(a.nbytes == b.nbytes for a, b in zip(olds, news))
        hdr = np.zeros(HEADER_BYTES, dtype=np.uint8)
        dbytes, pbytes = ctypes.c_uint64(0), ctypes.c_uint64(0)
        dcap = 1 << 16 if dir_cap is None else dir_cap
        pcap = 1 << 20 if payload_cap is None else payload_cap
        while True:
            d = np.zeros(max(dcap, 1), dtype=np.uint8)
            p = np.zeros(max(pcap, 1), dtype=np.uint8)
            rc = self.lib.orc_encode(T.ctypes.data, len(T), self._ptrs(olds), self._ptrs(news),
                                     sb.ctypes.data, len(olds), S.ctypes.data, len(S), mode,
                                     base_version, new_version, hdr.ctypes.data,
                                     d.ctypes.data, dcap, ctypes.byref(dbytes),
                                     p.ctypes.data, pcap, ctypes.byref(pbytes))
            if rc == E_CAPACITY and dir_cap is None and payload_cap is None:
                dcap, pcap = int(dbytes.value), int(pbytes.value)
                continue
            break
        if rc:
            return rc, hdr, d[:0], p[:0]
        return rc, hdr, d[: dbytes.value].copy(), p[: pbytes.value].copy()

    def encode_retry_partial(self, tensors, segments, old_shards, new_shards, delta_hdr, delta_dir,
                             delta_flags, base_version=0, new_version=1, dir_cap=None, payload_cap=None):
        """RETRY stream over the chunks with an unflagged DELTA record.
        Return (rc, header bytes, directory bytes, payload bytes)."""
        T = _pack(tensors, ORC_TENSOR)
        S = _pack(segments, ORC_SEGMENT)
        olds = [np.ascontiguousarray(s).view(np.uint8).reshape(-1) for s in old_shards]
        news = [np.ascontiguousarray(s).view(np.uint8).reshape(-1) for s in new_shards]
        sb = np.array([s.nbytes for s in olds], dtype=np.uint64)
        dh = np.ascontiguousarray(delta_hdr, dtype=np.uint8)
        dd = _nz(np.ascontiguousarray(delta_dir, dtype=np.uint8))
        df = _nz(np.ascontiguousarray(delta_flags, dtype=np.uint8))
        hdr = np.zeros(HEADER_BYTES, dtype=np.uint8)
        dbytes, pbytes = ctypes.c_uint64(0), ctypes.c_uint64(0)
        dcap = 1 << 16 if dir_cap is None else dir_cap
        pcap = 1 << 20 if payload_cap is None else payload_cap
        while True:
            d = np.zeros(max(dcap, 1), dtype=np.uint8)
            p = np.zeros(max(pcap, 1), dtype=np.uint8)
            rc = self.lib.orc_encode_retry_partial(T.ctypes.data, len(T), self._ptrs(olds), self._ptrs(news),
                                                   sb.ctypes.data, len(olds), S.ctypes.data, len(S),
                                                   dh.ctypes.data, dd.ctypes.data, df.ctypes.data,
                                                   base_version, new_version, hdr.ctypes.data,
                                                   d.ctypes.data, dcap, ctypes.byref(dbytes),
                                                   p.ctypes.data, pcap, ctypes.byref(pbytes))
            if rc == E_CAPACITY and dir_cap is None and payload_cap is None:
                dcap, pcap = int(dbytes.value), int(pbytes.value)
                continue
            break
        if rc:
            return rc, hdr, d[:0], p[:0]
        return rc, hdr, d[: dbytes.value].copy(), p[: pbytes.value].copy()

    def validate(self, tensors, hdr, d, p, expected_base_version=0, require_kind=-1) -> int:
        T = _pack(tensors, ORC_TENSOR)
        return int(self.lib.orc_validate(T.ctypes.data, len(T), hdr.ctypes.data,
                                         _nz(d).ctypes.data, _nz(p).ctypes.data,
                                         expected_base_version, require_kind))

    def apply(self, tensors, canon, hdr, d, p, flags, first=0, n=None,
              expected_base_version=0) -> int:
        """Apply records in place on the list of uint8 canonical arrays."""
        T = _pack(tensors, ORC_TENSOR)
        nrec = int(hdr[40:48].view("<u8")[0])
        n = nrec - first if n is None else n
        return int(self.lib.orc_apply(T.ctypes.data, len(T), self._ptrs(canon), hdr.ctypes.data,
                                      _nz(d).ctypes.data, _nz(p).ctypes.data, _nz(flags).ctypes.data,
                                      first, n, expected_base_version))

    def retry(self, tensors, canon, hdr, d, p, expected_base_version=0) -> int:
        T = _pack(tensors, ORC_TENSOR)
        return int(self.lib.orc_apply_overwrite_retry(
            T.ctypes.data, len(T), self._ptrs(canon), hdr.ctypes.data, _nz(d).ctypes.data,
            _nz(p).ctypes.data, expected_base_version))

    def apply_record_part(self, tensors, canon, d, p, rec, lo, hi) -> int:
        T = _pack(tensors, ORC_TENSOR)
        return int(self.lib.orc_apply_record_part(T.ctypes.data, len(T), self._ptrs(canon),
                                                  _nz(d).ctypes.data, _nz(p).ctypes.data,
                                                  rec, lo, hi))


def _transport(lib_fn, tensors, hdr, d, p):
    """Run orc_stream_pack / orc_stream_unpack; (rc, header, directory, payload)."""
    T = _pack(tensors, ORC_TENSOR)
    hdr = np.ascontiguousarray(hdr, dtype=np.uint8)
    d = np.ascontiguousarray(d, dtype=np.uint8)
    p = np.ascontiguousarray(p, dtype=np.uint8)
    ho = np.zeros(HEADER_BYTES, dtype=np.uint8)
    do = np.zeros(max(len(d), 1), dtype=np.uint8)
    need = ctypes.c_uint64(0)
    cap = 0
    while True:
        po = np.zeros(max(cap, 1), dtype=np.uint8)
        rc = lib_fn(T.ctypes.data, len(T), hdr.ctypes.data, _nz(d).ctypes.data, _nz(p).ctypes.data,
                    ho.ctypes.data, do.ctypes.data, po.ctypes.data, cap, ctypes.byref(need))
        if rc == E_CAPACITY and cap < int(need.value):
            cap = int(need.value)
            continue
        break
    if rc:
        return rc, ho, d[:0], p[:0]
    return rc, ho, do[: len(d)].copy(), po[: int(need.value)].copy()


def _pack_stream(self, tensors, hdr, d, p):
    """Transport packing (index-list records as gap varints)."""
    return _transport(self.lib.orc_stream_pack, tensors, hdr, d, p)


def _unpack_stream(self, tensors, hdr, d, p):
    """The inverse of pack_stream."""
    return _transport(self.lib.orc_stream_unpack, tensors, hdr, d, p)


Oracle.pack_stream = _pack_stream
Oracle.unpack_stream = _unpack_stream
LAYOUT_GAPS = 2
MAGIC_PACKED = 0x50524344


def _nz(a):
    """A non-empty array so that .ctypes.data is a valid pointer."""
    return a if a.size else np.zeros(1, dtype=np.uint8)


class OracleError(RuntimeError):
    def __init__(self, rc):
        super().__init__(f"oracle returned {rc}")
        self.rc = rc


_default = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
