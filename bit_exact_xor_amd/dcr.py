"""Python binding of libdcr.so (include/dcr.h): argument marshalling only.

Every step of encode / apply / retry runs in the library's gfx950 kernels;
this module packs descriptors into the C structs, turns torch tensors into
device pointers and the current torch stream into a hipStream_t, and raises
``DcrError`` on a nonzero status.  PyTorch provides device memory and streams.

The names follow the C-ABI: ``dcr_plan_build``, ``dcr_encode``,
``dcr_encode_retry_partial``, ``dcr_encode_retry_from_delta``, ``dcr_apply``,
``dcr_apply_overwrite_retry``, ``dcr_apply_sharded``, ``dcr_apply_overwrite_retry_sharded`` (plus the small
helpers around them).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdcr.so")

DCR_OK, DCR_E_INVAL, DCR_E_COVERAGE, DCR_E_FORMAT, DCR_E_VERSION, DCR_E_CAPACITY, DCR_E_HIP, DCR_E_NOMEM = \
    0, -1, -2, -3, -4, -5, -6, -7
DCR_E_TIMEOUT = -8
ROUTE_AFFINE_XOR, ROUTE_OVERWRITE, ROUTE_BLOCK_SCALED = 0, 1, 2
MODE_DELTA, MODE_RETRY = 0, 1
ENC_INDEX_LISTS = 0x100            # encode option: index-list layout for low-density records
LAYOUT_BITMAP, LAYOUT_LIST = 0, 1  # directory entry byte 15

# binary layouts of the C structs (include/dcr.h)
TENSOR_DESC = np.dtype([("numel", "<u8"), ("elem_bytes", "<u4"), ("route", "<u4"),
                        ("scale_tensor", "<i4"), ("scale_block", "<u4")])
SEGMENT = np.dtype([("tensor_id", "<u4"), ("shard_id", "<u4"), ("ndim", "<u4"), ("reserved", "<u4"),
                    ("shard_off", "<u8"), ("canon_off", "<u8"), ("extent", "<u8", (4,)),
                    ("shard_stride", "<i8", (4,)), ("canon_stride", "<i8", (4,))])
STREAM_HEADER = np.dtype([("magic", "<u4"), ("format_version", "<u2"), ("stream_kind", "<u2"),
                          ("chunk_bytes", "<u4"), ("reserved0", "<u4"), ("base_version", "<u8"),
                          ("new_version", "<u8"), ("plan_fingerprint", "<u8"), ("n_records", "<u8"),
                          ("payload_bytes", "<u8"), ("reserved1", "<u8")])
ENCODE_RESULT = np.dtype([("n_records", "<u8"), ("payload_bytes", "<u8"), ("n_changed", "<u8"),
                          ("status", "<i4"), ("n_reencoded", "<u4")])
APPLY_RESULT = np.dtype([("n_applied", "<u8"), ("n_skipped", "<u8"), ("n_invalid", "<u8"),
                         ("first_invalid", "<u8")])
assert TENSOR_DESC.itemsize == 24 and SEGMENT.itemsize == 128 and STREAM_HEADER.itemsize == 64
assert ENCODE_RESULT.itemsize == 32 and APPLY_RESULT.itemsize == 32


class PlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "n_tensors", "n_shards", "n_chunks", "n_pieces", "table_bytes", "workspace_bytes",
        "max_dir_bytes", "max_payload_bytes", "fingerprint", "canonical_bytes", "compact_stage_bytes")]


class DcrError(RuntimeError):
    def __init__(self, code: int, what: str, msg: str):
        super().__init__(f"{what} failed with {code}: {msg}")
        self.code = code


_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libdcr.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m bit_exact_xor_amd.build`")
    lib = ctypes.CDLL(p)
    P, U32, U64, I32 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int32
    lib.dcr_plan_build.restype = I32
    lib.dcr_plan_build.argtypes = [P, U32, P, U32, P, U64, ctypes.POINTER(P)]
    lib.dcr_plan_query.restype = I32
    lib.dcr_plan_query.argtypes = [P, ctypes.POINTER(PlanInfo)]
    lib.dcr_plan_upload.restype = I32
    lib.dcr_plan_upload.argtypes = [P, P, U64, P]
    lib.dcr_plan_destroy.restype = None
    lib.dcr_plan_destroy.argtypes = [P]
    lib.dcr_encode.restype = I32
    lib.dcr_encode.argtypes = [P, P, P, U32, U64, U64, P, P, U64, P, U64, P, P, U64, P]
    lib.dcr_encode_pipelined.restype = I32
    for fn in (lib.dcr_stream_pack, lib.dcr_stream_unpack):
        fn.restype = I32
        fn.argtypes = [P, P, P, P, P, P, U64, P, U64, P, P, U64, P]
    lib.dcr_encode_noalloc.restype = I32
    lib.dcr_encode_noalloc.argtypes = [P, P, P, U32, U64, U64, P, P, U64, P, U64, P, P]
    lib.dcr_encode_pipelined.argtypes = [P, P, P, U32, U64, U64, P, P, U64, P, U64, P, P, U64, U32, P, U64, P]
    lib.dcr_ready_wait.restype = I32
    lib.dcr_ready_wait.argtypes = [P, U32, U64, P]
    lib.dcr_encode_retry_partial.restype = I32
    lib.dcr_encode_retry_partial.argtypes = [P, P, P, P, P, U64, P, U64, U64, P, P, U64, P, U64, P, P, U64, P]
    lib.dcr_encode_retry_from_delta.restype = I32
    lib.dcr_encode_retry_from_delta.argtypes = [P, P, P, P, U64, P, U64, U32, P, P, U64, P, U64, P, P, U64, P]
    lib.dcr_apply.restype = I32
    lib.dcr_apply.argtypes = [P, P, P, P, P, P, U64, U64, U64, P, P, U64, P]
    lib.dcr_apply_sharded.restype = I32
    lib.dcr_apply_sharded.argtypes = [P, P, P, P, P, P, U64, U64, U64, P, P, U64, P]
    lib.dcr_apply_overwrite_retry_sharded.restype = I32
    lib.dcr_apply_overwrite_retry_sharded.argtypes = [P, P, P, P, P, U64, P, P, U64, P]
    lib.dcr_apply_overwrite_retry.restype = I32
    lib.dcr_apply_overwrite_retry.argtypes = [P, P, P, P, P, U64, P, P, U64, P]
    lib.dcr_last_error.restype = ctypes.c_char_p
    lib.dcr_last_error.argtypes = []
    lib.dcr_set_kernel_events.restype = None
    lib.dcr_set_kernel_events.argtypes = [P, P]
    lib.dcr_format_constants.restype = U32
    lib.dcr_format_constants.argtypes = [P, U32]
    if path is None:
        _lib = lib
    return lib


def _check(rc: int, what: str) -> None:
    if rc != DCR_OK:
        raise DcrError(rc, what, load_library().dcr_last_error().decode())


def _pack(arr, dtype):
    out = np.zeros(len(arr), dtype=dtype)
    for name in dtype.names:
        if name == "reserved":
            continue
        out[name] = arr[name]
    return out


def _ptr_array(ptrs):
    arr = (ctypes.c_void_p * max(1, len(ptrs)))()
    for i, p in enumerate(ptrs):
        arr[i] = int(p) if p else None
    return arr


class PtrTable:
    """The device addresses of a fixed list of buffers (shards or canonical
    tensors), packed once into pinned host memory.  Pass it wherever a list
    of buffers is taken: calls on plans with many tensors then skip
    rebuilding the address array, and the library's copy of it to the
    workspace is an asynchronous DMA instead of a staged pageable copy.  The
    buffers are kept alive by the table; it must not outlive their storage
    moving (torch never moves a tensor's storage).  Needs a GPU runtime
    (pinned host memory); a table passed to calls captured into a HIP graph
    must outlive the graph, whose copy nodes read it at every replay."""

    def __init__(self, bufs):
        import torch
        self.bufs = list(bufs)
        n = len(self.bufs)
        self.host = torch.empty(max(1, n), dtype=torch.int64, pin_memory=True)
        if n:
            self.host.numpy()[:n] = np.array([_dptr(t) for t in self.bufs], dtype=np.uint64).view(np.int64)
        self.address = int(self.host.data_ptr())

    def __len__(self):
        return len(self.bufs)


def _ptrs(bufs):
    """A C array of device addresses for a list of buffers or a PtrTable."""
    if isinstance(bufs, PtrTable):
        return ctypes.c_void_p(bufs.address)
    return _ptr_array([_dptr(t) for t in bufs])


def _dptr(t) -> int:
    """Device pointer of a torch tensor (or an int address)."""
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return int(t.ctypes.data)
    return int(t.data_ptr())


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream or None
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else (int(stream) or None)


class Plan:
    """A built plan (host) plus its device tables once uploaded."""

    def __init__(self, handle: int, info: PlanInfo):
        self.handle = handle
        self.info = info
        self.tables = None

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h and _lib is not None:
            _lib.dcr_plan_destroy(h)


def dcr_plan_build(tensors, shard_bytes, segments) -> Plan:
    """Build a plan from a tensor table, shard sizes (bytes) and affine segments."""
    lib = load_library()
    T = _pack(tensors, TENSOR_DESC)
    S = _pack(segments, SEGMENT)
    sb = np.ascontiguousarray(np.asarray(shard_bytes, dtype=np.uint64))
    h = ctypes.c_void_p()
    rc = lib.dcr_plan_build(T.ctypes.data if len(T) else None, len(T), sb.ctypes.data if len(sb) else None,
                            len(sb), S.ctypes.data if len(S) else None, len(S), ctypes.byref(h))
    _check(rc, "dcr_plan_build")
    info = PlanInfo()
    _check(lib.dcr_plan_query(h, ctypes.byref(info)), "dcr_plan_query")
    return Plan(h.value, info)


def dcr_plan_upload(plan: Plan, device="cuda", stream=None) -> None:
    import torch
    plan.tables = torch.empty(max(int(plan.info.table_bytes), 16), dtype=torch.uint8, device=device)
    _check(load_library().dcr_plan_upload(plan.handle, plan.tables.data_ptr(), plan.tables.numel(),
                                          _stream(stream)), "dcr_plan_upload")


def dcr_encode(plan: Plan, old_shards, new_shards, mode, base_version, new_version,
               header, dir_buf, payload, result, workspace, stream=None) -> None:
    """Enqueue an encode; buffers are torch device tensors (or int addresses)."""
    rc = load_library().dcr_encode(
        plan.handle, _ptrs(old_shards), _ptrs(new_shards),
        mode, base_version, new_version, _dptr(header), _dptr(dir_buf), _nbytes(dir_buf), _dptr(payload),
        _nbytes(payload), _dptr(result), _dptr(workspace), _nbytes(workspace), _stream(stream))
    _check(rc, "dcr_encode")


LAYOUT_GAPS = 2                    # directory entry byte 15, packed streams only
MAGIC_PACKED = 0x50524344


def _transport(fn, what, plan, header, dir_buf, payload, header_out, dir_out, payload_out, result, workspace,
               stream=None):
    h = np.ascontiguousarray(np.asarray(header, dtype=np.uint8).reshape(-1)[:64])
    rc = fn(plan.handle, h.ctypes.data, _dptr(dir_buf), _dptr(payload), _dptr(header_out), _dptr(dir_out),
            _nbytes(dir_out), _dptr(payload_out), _nbytes(payload_out), _dptr(result), _dptr(workspace),
            _nbytes(workspace), _stream(stream))
    _check(rc, what)


def dcr_stream_pack(plan: Plan, header, dir_buf, payload, header_out, dir_out, payload_out, result, workspace,
                    stream=None) -> None:
    """Enqueue the transport packing of a stream (host header, device
    buffers) into the output buffers."""
    _transport(load_library().dcr_stream_pack, "dcr_stream_pack", plan, header, dir_buf, payload, header_out,
               dir_out, payload_out, result, workspace, stream)


def dcr_stream_unpack(plan: Plan, header, dir_buf, payload, header_out, dir_out, payload_out, result, workspace,
                      stream=None) -> None:
    """Enqueue the inverse of dcr_stream_pack."""
    _transport(load_library().dcr_stream_unpack, "dcr_stream_unpack", plan, header, dir_buf, payload, header_out,
               dir_out, payload_out, result, workspace, stream)


NOALLOC_SCRATCH_BYTES = 64 << 20   # DCR_NOALLOC_SCRATCH_BYTES


def dcr_encode_noalloc(plan: Plan, old_shards, new_shards, mode, base_version, new_version,
                       header, dir_buf, payload, result, stream=None) -> None:
    """Enqueue an encode that uses the library's own device scratch array as
    its workspace (no workspace argument; calls overlapping on one GPU race)."""
    rc = load_library().dcr_encode_noalloc(
        plan.handle, _ptrs(old_shards), _ptrs(new_shards),
        mode, base_version, new_version, _dptr(header), _dptr(dir_buf), _nbytes(dir_buf), _dptr(payload),
        _nbytes(payload), _dptr(result), _stream(stream))
    _check(rc, "dcr_encode_noalloc")


def ready_region_bytes(n_slices: int) -> int:
    """Bytes of a dcr_encode_pipelined watermark region for n_slices."""
    return 64 + 64 * int(n_slices)


def dcr_encode_pipelined(plan: Plan, old_shards, new_shards, mode, base_version, new_version,
                         header, dir_buf, payload, result, workspace, n_slices, ready, stream=None) -> None:
    """Enqueue a sliced encode that publishes a ready watermark after each
    slice into `ready`, a pinned host tensor of ready_region_bytes(n_slices)."""
    rc = load_library().dcr_encode_pipelined(
        plan.handle, _ptrs(old_shards), _ptrs(new_shards),
        mode, base_version, new_version, _dptr(header), _dptr(dir_buf), _nbytes(dir_buf), _dptr(payload),
        _nbytes(payload), _dptr(result), _dptr(workspace), _nbytes(workspace), n_slices, _dptr(ready),
        _nbytes(ready), _stream(stream))
    _check(rc, "dcr_encode_pipelined")


def dcr_ready_wait(ready, slice_index: int, timeout_us: int = 10_000_000) -> np.ndarray:
    """Wait until slice `slice_index` of a watermark region is published;
    returns its prefix header (64 bytes)."""
    out = np.zeros(64, dtype=np.uint8)
    rc = load_library().dcr_ready_wait(_dptr(ready), slice_index, timeout_us, out.ctypes.data)
    _check(rc, "dcr_ready_wait")
    return out


def dcr_encode_retry_partial(plan: Plan, old_shards, new_shards, delta_header: np.ndarray, delta_dir, delta_flags,
                             base_version, new_version, header, dir_buf, payload, result, workspace,
                             stream=None) -> None:
    """Enqueue a partial retry encode: a RETRY stream over the chunks that hold
    a record of the DELTA stream (host header bytes, device directory) whose
    applied flag (device bytes) is 0."""
    hdr = np.ascontiguousarray(np.asarray(delta_header, dtype=np.uint8))
    rc = load_library().dcr_encode_retry_partial(
        plan.handle, _ptrs(old_shards), _ptrs(new_shards),
        hdr.ctypes.data, _dptr(delta_dir), _nbytes(delta_dir), _dptr(delta_flags), base_version, new_version,
        _dptr(header), _dptr(dir_buf), _nbytes(dir_buf), _dptr(payload), _nbytes(payload), _dptr(result),
        _dptr(workspace), _nbytes(workspace), _stream(stream))
    _check(rc, "dcr_encode_retry_partial")


def dcr_encode_retry_from_delta(plan: Plan, old_shards, delta_header: np.ndarray, delta_dir, delta_payload,
                                options, header, dir_buf, payload, result, workspace, stream=None) -> None:
    """Enqueue a RETRY stream written from a DELTA stream (host header bytes,
    device directory and payload) and the old shards; options 0 or
    DCR_ENC_INDEX_LISTS."""
    hdr = np.ascontiguousarray(np.asarray(delta_header, dtype=np.uint8))
    rc = load_library().dcr_encode_retry_from_delta(
        plan.handle, _ptrs(old_shards), hdr.ctypes.data, _dptr(delta_dir), _nbytes(delta_dir),
        _dptr(delta_payload), _nbytes(delta_payload), options, _dptr(header), _dptr(dir_buf), _nbytes(dir_buf),
        _dptr(payload), _nbytes(payload), _dptr(result), _dptr(workspace), _nbytes(workspace), _stream(stream))
    _check(rc, "dcr_encode_retry_from_delta")


def dcr_apply(plan: Plan, canon, header: np.ndarray, dir_buf, payload, flags, first_record, n_records,
              expected_base_version, result, workspace, stream=None) -> None:
    """Enqueue an apply of records [first, first+n); header is host bytes (64)."""
    hdr = np.ascontiguousarray(np.asarray(header, dtype=np.uint8))
    rc = load_library().dcr_apply(
        plan.handle, _ptrs(canon), hdr.ctypes.data, _dptr(dir_buf), _dptr(payload),
        _dptr(flags), first_record, n_records, expected_base_version, _dptr(result), _dptr(workspace),
        _nbytes(workspace), _stream(stream))
    _check(rc, "dcr_apply")


def dcr_apply_overwrite_retry(plan: Plan, canon, header: np.ndarray, dir_buf, payload,
                              expected_base_version, result, workspace, stream=None) -> None:
    hdr = np.ascontiguousarray(np.asarray(header, dtype=np.uint8))
    rc = load_library().dcr_apply_overwrite_retry(
        plan.handle, _ptrs(canon), hdr.ctypes.data, _dptr(dir_buf), _dptr(payload),
        expected_base_version, _dptr(result), _dptr(workspace), _nbytes(workspace), _stream(stream))
    _check(rc, "dcr_apply_overwrite_retry")


def dcr_apply_sharded(plan: Plan, shards, header: np.ndarray, dir_buf, payload, flags, first_record, n_records,
                      expected_base_version, result, workspace, stream=None) -> None:
    """Apply records [first, first+n) into a receiver layout: `plan` is the
    receiver plan, `shards` its device shards."""
    hdr = np.ascontiguousarray(np.asarray(header, dtype=np.uint8))
    rc = load_library().dcr_apply_sharded(
        plan.handle, _ptrs(shards), hdr.ctypes.data, _dptr(dir_buf), _dptr(payload),
        _dptr(flags), first_record, n_records, expected_base_version, _dptr(result), _dptr(workspace),
        _nbytes(workspace), _stream(stream))
    _check(rc, "dcr_apply_sharded")


def dcr_apply_overwrite_retry_sharded(plan: Plan, shards, header: np.ndarray, dir_buf, payload,
                                      expected_base_version, result, workspace, stream=None) -> None:
    """Overwrite retry into a receiver layout (see dcr_apply_sharded)."""
    hdr = np.ascontiguousarray(np.asarray(header, dtype=np.uint8))
    rc = load_library().dcr_apply_overwrite_retry_sharded(
        plan.handle, _ptrs(shards), hdr.ctypes.data, _dptr(dir_buf), _dptr(payload),
        expected_base_version, _dptr(result), _dptr(workspace), _nbytes(workspace), _stream(stream))
    _check(rc, "dcr_apply_overwrite_retry_sharded")


def dcr_set_kernel_events(start=None, stop=None) -> None:
    """Record start / stop (torch.cuda.Event, created, or raw hipEvent_t) around
    the main kernel of the following calls on this thread; None, None: off."""
    def h(e):
        if e is None:
            return None
        return int(e.cuda_event) if hasattr(e, "cuda_event") else int(e)
    load_library().dcr_set_kernel_events(h(start), h(stop))


def format_constants():
    out = (ctypes.c_uint32 * 10)()
    n = load_library().dcr_format_constants(out, 10)
    return list(out)[:n]


def _nbytes(t) -> int:
    if isinstance(t, np.ndarray):
        return int(t.nbytes)
    return int(t.numel() * t.element_size()) if hasattr(t, "numel") else 0


# ------------------------------------------------------- small conveniences

class StreamBuffers:
    """Device buffers of one stream (header, directory, payload, result)."""

    def __init__(self, plan: Plan, device="cuda", dir_bytes=None, payload_bytes=None):
        import torch
        self.header = torch.zeros(64, dtype=torch.uint8, device=device)
        self.dir = torch.empty(max(int(dir_bytes if dir_bytes is not None else plan.info.max_dir_bytes), 32),
                               dtype=torch.uint8, device=device)
        self.payload = torch.empty(max(int(payload_bytes if payload_bytes is not None
                                           else plan.info.max_payload_bytes), 16),
                                   dtype=torch.uint8, device=device)
        self.result = torch.zeros(32, dtype=torch.uint8, device=device)

    def header_host(self) -> np.ndarray:
        return self.header.cpu().numpy()

    def result_host(self):
        return np.frombuffer(self.result.cpu().numpy().tobytes(), dtype=ENCODE_RESULT)[0]

    def n_records(self) -> int:
        return int(self.result_host()["n_records"])

    def payload_bytes(self) -> int:
        return int(self.result_host()["payload_bytes"])


def workspace(plan: Plan, device="cuda", stage_bytes: int = 0):
    """Workspace of the plan's size plus an optional encode staging area."""
    import torch
    return torch.zeros(max(int(plan.info.workspace_bytes) + int(stage_bytes), 256), dtype=torch.uint8,
                       device=device)


def apply_result(t) -> np.void:
    return np.frombuffer(t.cpu().numpy().tobytes(), dtype=APPLY_RESULT)[0]
