/*
 * dcr.h -- C-ABI of the MI355X (gfx950) bit-exact delta encode / apply library.
 *
 * The library implements the data-parallel core of bit-exact delta-compressed
 * refit as described on the NeMo-DCR pages:
 *   - the owner of each training shard compares new against the last committed
 *     weights on their stored bits, not as float values, so +0/-0 and other
 *     sign flips are changes (ai-feeds summary "Method / input and change
 *     detection"; tokendh blog "shard owner");
 *   - changed elements are projected by a fixed affine map from the shard's
 *     local index to canonical checkpoint coordinates (ai-feeds summary "key
 *     modules" 1; ai.info abstract); non-affine ones (fused QKV, shared
 *     scales) become overwrite records (ai-feeds "key modules" 2; tokendh
 *     "shard owner");
 *   - affine changes travel as XOR masks, the rest as overwrites, in one delta
 *     stream (ai-feeds "key modules" 2-3; tokendh "XOR or overwrite"); the
 *     delta algebra is mask = old ^ new, new = old ^ mask on a flat bit buffer
 *     (humansand "weight teleportation" page, "Delta update algebra");
 *   - the receiver applies the records in place with per-record dedup flags,
 *     since a XOR applied twice undoes itself (tokendh "XOR or overwrite"), and
 *     a retry re-applies the whole change set as overwrites, which is
 *     idempotent (tokendh "no backup copy"; ai.info abstract).
 *
 * Record format (the pages fix none; this is the library's own): per 64 KiB
 * chunk of each canonical tensor, at most one XOR and one overwrite record,
 * each = change bitmap | low byte plane | upper planes, every section
 * zero-padded to 16 bytes; XOR records on 2-byte elements elide zero high
 * bytes with a presence bitmap when that is strictly smaller (SPARSE), keep
 * all high bytes otherwise (DENSE) or none when all are zero (NONE).  A
 * 64-byte stream header and 32-byte directory entries describe the stream.
 * Encoded with DCR_ENC_INDEX_LISTS, a record whose K changes take fewer bytes
 * as 16-bit element indices (padded) than as its padded bitmap carries the
 * ascending indices in the bitmap's place, marked in byte 15 of its directory
 * entry (DCR_LAYOUT_LIST); the mask stream is sparse and worth compressing
 * (ai-feeds "key modules" 3).
 *
 * Conventions
 *   - All integers little-endian.  All status codes: 0 = DCR_OK, < 0 = error.
 *   - Host-detectable errors are returned synchronously; the message is in
 *     dcr_last_error() (thread-local).  Device-detected conditions (capacity,
 *     invalid records) are reported in result structs in device memory.
 *   - Memory: the caller owns ALL device memory (shards, canonical tensors,
 *     directory, payload, flags, workspace, plan tables).  The library
 *     allocates host memory only (the plan) and never calls hipMalloc.
 *   - Streams: `stream` is a hipStream_t (NULL = the null stream).  All device
 *     work is enqueued on it; the library never synchronises it.  Host arrays
 *     of device pointers passed to a call are copied to the workspace by an
 *     asynchronous copy on `stream`: from pageable memory the copy has read
 *     the array when the call returns; from pinned memory (hipHostMalloc) it
 *     reads it when the stream reaches it, so the array must stay unchanged
 *     until then.
 *   - Graph capture: the calls enqueue only kernels and those pointer-array
 *     copies (no memset, allocation or synchronisation), so they may be
 *     captured into a HIP graph.  A captured copy reads its host array at
 *     every replay: pass pinned arrays that outlive the graph.  Sizes, plan
 *     and stream header are fixed at capture.
 *   - Alignment: every shard, canonical tensor, directory, payload, result and
 *     workspace pointer must be 16-byte aligned (DCR_E_INVAL otherwise).
 *   - Concurrency: a plan is immutable after upload and may be shared; calls
 *     that run concurrently need separate workspaces.
 */
#ifndef DCR_H
#define DCR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ constants */
enum {
    DCR_OK = 0,
    DCR_E_INVAL = -1,     /* bad argument / descriptor / alignment            */
    DCR_E_COVERAGE = -2,  /* canonical elements not covered exactly once      */
    DCR_E_FORMAT = -3,    /* stream header does not match (magic, plan, kind) */
    DCR_E_VERSION = -4,   /* stream base_version != expected base version     */
    DCR_E_CAPACITY = -5,  /* a caller buffer is too small                     */
    DCR_E_HIP = -6,       /* a HIP runtime call failed                        */
    DCR_E_NOMEM = -7,     /* host allocation failed                           */
    DCR_E_TIMEOUT = -8    /* dcr_ready_wait: slice not published in time      */
};
enum { DCR_ROUTE_AFFINE_XOR = 0, DCR_ROUTE_OVERWRITE = 1, DCR_ROUTE_BLOCK_SCALED = 2 };
enum { DCR_MODE_DELTA = 0, DCR_MODE_RETRY = 1 };
/* encode option, OR-ed into dcr_encode's mode: index-list layout for records
 * where it is smaller than the bitmap (the stream kind stays mode & 0xFF) */
enum { DCR_ENC_INDEX_LISTS = 0x100 };
/* record layouts (byte 15 of a directory entry); DCR_LAYOUT_GAPS only in a
 * packed stream (dcr_stream_pack) */
enum { DCR_LAYOUT_BITMAP = 0, DCR_LAYOUT_LIST = 1, DCR_LAYOUT_GAPS = 2 };
enum { DCR_KIND_XOR = 0, DCR_KIND_OW = 1 };
enum { DCR_HI_NONE = 0, DCR_HI_SPARSE = 1, DCR_HI_DENSE = 2 };
#define DCR_MAGIC 0x31524344u          /* "DCR1" */
#define DCR_MAGIC_PACKED 0x50524344u   /* "DCRP": a packed stream (dcr_stream_pack) */
#define DCR_FORMAT_VERSION 1u
#define DCR_CHUNK_BYTES 65536u
#define DCR_HEADER_BYTES 64u
#define DCR_DIRENT_BYTES 32u

/* ---------------------------------------------------------------- types */

/* One canonical (checkpoint) tensor.  24 bytes.
 *   numel        elements
 *   elem_bytes   1, 2 or 4 (XOR-carrying routes: 1 or 2 only)
 *   route        DCR_ROUTE_*: AFFINE_XOR -> XOR records; OVERWRITE -> overwrite
 *                records; BLOCK_SCALED -> an element is an overwrite iff the
 *                fp32 bits of its block's scale changed, else XOR
 *   scale_tensor BLOCK_SCALED: id of its fp32 OVERWRITE scale tensor, which
 *                has ceil(numel / scale_block) elements; else -1
 *   scale_block  BLOCK_SCALED: elements per scale, a multiple of 16/elem_bytes;
 *                else 0 */
typedef struct {
    uint64_t numel;
    uint32_t elem_bytes;
    uint32_t route;
    int32_t scale_tensor;
    uint32_t scale_block;
} dcr_tensor_desc;

/* One affine segment of the direct projection: for every multi-index x with
 * 0 <= x_d < extent[d] (d < ndim, 1 <= ndim <= 4), canonical element
 *   canon_off + sum_d x_d * canon_stride[d]   of tensor tensor_id
 * is stored at element
 *   shard_off + sum_d x_d * shard_stride[d]   of shard shard_id,
 * in element units of the tensor's width.  128 bytes.  Every canonical
 * element must be covered exactly once over all segments. */
typedef struct {
    uint32_t tensor_id, shard_id, ndim, reserved;
    uint64_t shard_off, canon_off;
    uint64_t extent[4];
    int64_t shard_stride[4];
    int64_t canon_stride[4];
} dcr_segment;

typedef struct dcr_plan dcr_plan; /* opaque; host-owned */

typedef struct {
    uint64_t n_tensors, n_shards, n_chunks, n_pieces;
    uint64_t table_bytes;       /* device bytes dcr_plan_upload needs            */
    uint64_t workspace_bytes;   /* device workspace bytes encode / apply need    */
    uint64_t max_dir_bytes;     /* directory bytes of the largest possible stream */
    uint64_t max_payload_bytes; /* payload bytes of the largest possible stream
                                   (each chunk's worst case, 16-aligned); also
                                   the size of encode's staging area          */
    uint64_t fingerprint;       /* FNV-1a-64 of the serialised tensor table       */
    uint64_t canonical_bytes;   /* sum of numel * elem_bytes                      */
    uint64_t compact_stage_bytes; /* the least staging area dcr_encode uses
                                   compactly: 1/16 of max_payload_bytes
                                   (16-byte aligned, at least 1 KiB); below
                                   it the encode runs in order                */
} dcr_plan_info;

/* Stream header, 64 bytes (the first bytes of every stream). */
typedef struct {
    uint32_t magic;             /* DCR_MAGIC */
    uint16_t format_version;    /* DCR_FORMAT_VERSION */
    uint16_t stream_kind;       /* DCR_MODE_DELTA or DCR_MODE_RETRY */
    uint32_t chunk_bytes;       /* 65536 */
    uint32_t reserved0;
    uint64_t base_version;
    uint64_t new_version;
    uint64_t plan_fingerprint;
    uint64_t n_records;
    uint64_t payload_bytes;
    uint64_t reserved1;
} dcr_stream_header;

/* Written by dcr_encode in device memory.  32 bytes. */
typedef struct {
    uint64_t n_records;         /* records of the stream (also when it did not fit) */
    uint64_t payload_bytes;     /* payload bytes of the stream (also when it did not fit) */
    uint64_t n_changed;         /* elements whose stored bits differ */
    int32_t status;             /* DCR_OK, or DCR_E_CAPACITY if dir_cap / payload_cap
                                   was too small: grow the buffers and encode again;
                                   DCR_E_FORMAT from dcr_encode_retry_partial if the
                                   DELTA directory names a chunk the plan lacks */
    uint32_t n_reencoded;       /* chunks encoded a second time because a compact
                                   staging area had no room left for them (0 with
                                   a full staging area or none) */
} dcr_encode_result;

/* Written by dcr_apply / dcr_apply_overwrite_retry in device memory.  32 bytes. */
typedef struct {
    uint64_t n_applied;         /* records applied by this call */
    uint64_t n_skipped;         /* records skipped because their flag was set */
    uint64_t n_invalid;         /* records refused (malformed entry or payload); untouched */
    uint64_t first_invalid;     /* lowest refused record index, or UINT64_MAX */
} dcr_apply_result;

/* --------------------------------------------------------------- calls */

/* Build a plan from the canonical tensor table, the shard sizes (bytes) and
 * the affine segments (see dcr_segment).
 * Passages: a fixed affine map that depends only on the static shard layout
 * projects a shard-local index to canonical checkpoint coordinates (ai-feeds
 * summary "key modules" 1, direct projection); each training shard has one
 * owner, so replicas are checked once (tokendh blog "shard owner"); ownership
 * is remapped so that the ranks cover the checkpoint exactly once and the
 * tiling / address metadata is prepared on the CPU (humansand "weight
 * teleportation" page, "A strong baseline with Blackwell-native DE").  Checks every descriptor, that every
 * segment stays inside its tensor and shard (DCR_E_INVAL) and that every
 * canonical element is covered exactly once (DCR_E_COVERAGE; the ownership
 * invariant: one owner per element, replicas are not listed).  Expands the
 * segments into contiguous runs, cuts them at 64 KiB canonical chunk borders
 * and builds the chunk and piece tables the kernels read.  On success *out
 * owns host memory; free it with dcr_plan_destroy. */
int32_t dcr_plan_build(const dcr_tensor_desc* tensors, uint32_t n_tensors,
                       const uint64_t* shard_bytes, uint32_t n_shards,
                       const dcr_segment* segments, uint64_t n_segments,
                       dcr_plan** out);

/* Sizes and fingerprint of a plan. */
int32_t dcr_plan_query(const dcr_plan* plan, dcr_plan_info* out);

/* Copy the plan's tables to caller-owned device memory `dev_tables` (at least
 * table_bytes, 16-byte aligned) on `stream`, and bind the plan to it.  The
 * memory must stay allocated and unmodified while the plan is used.  The host
 * copy source is owned by the plan, which must outlive the copy. */
int32_t dcr_plan_upload(dcr_plan* plan, void* dev_tables, uint64_t bytes, void* stream);

void dcr_plan_destroy(dcr_plan* plan);

/* Encode one refit step (sender side).
 * Passages: the owner of each training shard detects the weights whose stored
 * value changed since the last version (ai-feeds summary "Method / input and
 * change detection"), comparing stored bit patterns rather than float values,
 * so +0/-0 and other sign flips count (tokendh blog "shard owner"); affine
 * changes are projected to canonical coordinates and carried as XOR masks,
 * the residual ones (fused QKV, shared scales) as overwrites, both in one
 * delta stream (ai-feeds "key modules" 1-3; tokendh "XOR or overwrite");
 * mask = old ^ new on a flat bit buffer (humansand "weight teleportation"
 * page, "Delta update algebra").
 *   old_shards / new_shards  host arrays of n_shards device pointers: the
 *                  trainer shards of the committed base and of the new step
 *   mode           DCR_MODE_DELTA: XOR / overwrite records by route;
 *                  DCR_MODE_RETRY: one overwrite record per changed chunk
 *                  carrying the new stored bits of every changed element;
 *                  either OR DCR_ENC_INDEX_LISTS: low-density records in the
 *                  index-list layout (default: every record carries a bitmap)
 *   base_version, new_version  written to the header (version binding)
 *   header_dev     64 bytes of device memory for the stream header
 *   dir_dev, dir_cap           directory buffer and its size in bytes
 *   payload_dev, payload_cap   payload buffer and its size in bytes
 *   result_dev     a dcr_encode_result in device memory
 *   workspace_dev, ws_bytes    at least workspace_bytes of device memory.
 *                  The excess past workspace_bytes is a staging area.  With
 *                  at least max_payload_bytes of it, each chunk writes its
 *                  records to a slot of its own (sized for its worst case)
 *                  at once and a second pass moves them into place, so no
 *                  chunk waits for another.  With less, but at least
 *                  compact_stage_bytes (dcr_encode_pipelined excepted), the
 *                  area is used compactly: it is cut into 64 partitions and
 *                  each chunk claims exactly its records' bytes in one of
 *                  them (one atomic add); a chunk that finds no room is
 *                  encoded again, straight to its place, after the offsets
 *                  are known.  An area a little larger than the stream's
 *                  payload runs at nearly the speed of the whole worst case;
 *                  one far below it encodes most chunks twice, slower than
 *                  in order (size the area from the last stream's
 *                  payload_bytes).  With less than compact_stage_bytes, or
 *                  none, each chunk waits until every earlier
 *                  chunk has published its sizes (decoupled look-back) and
 *                  writes in place.  All give the same stream.
 * Records are written in (tensor, chunk, kind) order with contiguous 16-byte
 * aligned payload offsets.  If a buffer is too small, result->status becomes
 * DCR_E_CAPACITY with the required totals; the buffers then hold no usable
 * stream.  Read the result after synchronising the stream. */
int32_t dcr_encode(const dcr_plan* plan,
                   const void* const* old_shards, const void* const* new_shards,
                   uint32_t mode, uint64_t base_version, uint64_t new_version,
                   void* header_dev, void* dir_dev, uint64_t dir_cap,
                   void* payload_dev, uint64_t payload_cap,
                   dcr_encode_result* result_dev,
                   void* workspace_dev, uint64_t ws_bytes, void* stream);

/* Allocation-free encode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): dcr_encode without a workspace argument.  The workspace and the
 * staging area live in a device array of the library, DCR_NOALLOC_SCRATCH_BYTES
 * on each GPU, held from the library's first use on that GPU until the process
 * ends; its address on the current device is looked up once per device.  The
 * encode runs staged when workspace_bytes + max_payload_bytes fit the array,
 * else in order (decoupled look-back, no staging); the stream is the same as
 * dcr_encode's.  The call allocates nothing (no hipMalloc; on the host only
 * the error text) and enqueues the same kind of work as dcr_encode.
 *   Errors: DCR_E_CAPACITY, before anything is enqueued, when the plan's
 *   workspace_bytes exceed DCR_NOALLOC_SCRATCH_BYTES; otherwise as dcr_encode.
 *   Concurrency: every call on one GPU uses that GPU's one array, and the
 *   array keeps the last call's contents (each call clears what it needs
 *   cleared), so calls that overlap on one GPU (other streams or threads)
 *   race and must be serialised by the caller.  Other entry points do not
 *   touch the array. */
#define DCR_NOALLOC_SCRATCH_BYTES (64u << 20)
int32_t dcr_encode_noalloc(const dcr_plan* plan,
                           const void* const* old_shards, const void* const* new_shards,
                           uint32_t mode, uint64_t base_version, uint64_t new_version,
                           void* header_dev, void* dir_dev, uint64_t dir_cap,
                           void* payload_dev, uint64_t payload_cap,
                           dcr_encode_result* result_dev, void* stream);

/* Pipelined encode (sender side): the trainer starts sending finished parts
 * of the stream while the rest is still being built, so a refit costs about
 * the larger of build and transfer time rather than their sum (ai-feeds
 * summary "key modules" 5, pipelined transfer; tokendh blog, the paragraph
 * on pipelining build and transfer).  Same arguments and the same stream as
 * dcr_encode, plus a ready watermark:
 *   n_slices       the encode runs as this many slices in plan (tensor,
 *                  chunk) order; at most one per 256 chunks of the plan
 *                  (fewer are used if asked for more; at least 1).  With
 *                  nb = ceil(n_chunks / 256), slice k covers the plan's chunks
 *                  [256 * floor(k * nb / n), min(256 * floor((k + 1) * nb / n),
 *                  n_chunks)), n the slices used.
 *   ready_host     the watermark region, 64 + 64 * n_slices bytes of pinned
 *                  host memory (hipHostMalloc), 64-byte aligned; anything else
 *                  is refused (DCR_E_INVAL) before any launch.  Layout:
 *                    u64 @0   slices published so far (0 .. n), monotone
 *                    i32 @8   0, or the stream's failure status once the
 *                             stream stops fitting its buffers
 *                             (DCR_E_CAPACITY) or a partial-retry directory
 *                             is bad (DCR_E_FORMAT); nothing more is then
 *                             published
 *                    u32 @12  n, the slices used
 *                    @64 + 64 k  prefix header k: the stream header of the
 *                             stream cut after slice k (its n_records and
 *                             payload_bytes count the records of chunks
 *                             before the slice's end)
 *                  This call resets @0 and @8 and sets @12 from the host; the
 *                  region must not be in use by an encode still in flight.
 *   ready_bytes    size of that region.
 * Once slice k is published, directory entries [0, prefix[k].n_records) and
 * payload bytes [0, prefix[k].payload_bytes) are final in device memory and
 * may be copied out by any stream or engine while the encode goes on; the
 * prefix is itself a valid stream, so a receiver may apply records
 * [prefix[k-1].n_records, prefix[k].n_records) with prefix header k
 * (dcr_apply) as they arrive.  When slice n - 1 is published, header_dev and
 * result_dev are final too and prefix header n - 1 equals the header. */
int32_t dcr_encode_pipelined(const dcr_plan* plan,
                             const void* const* old_shards, const void* const* new_shards,
                             uint32_t mode, uint64_t base_version, uint64_t new_version,
                             void* header_dev, void* dir_dev, uint64_t dir_cap,
                             void* payload_dev, uint64_t payload_cap,
                             dcr_encode_result* result_dev,
                             void* workspace_dev, uint64_t ws_bytes,
                             uint32_t n_slices, void* ready_host, uint64_t ready_bytes,
                             void* stream);

/* Wait (host side, polling; no HIP call) until slice `slice` of a
 * dcr_encode_pipelined watermark region is published and copy its prefix
 * header to `out`.  Returns DCR_OK; the region's failure status if the encode
 * stopped publishing; DCR_E_TIMEOUT after timeout_us microseconds;
 * DCR_E_INVAL for a slice beyond the region's count. */
int32_t dcr_ready_wait(const void* ready_host, uint32_t slice, uint64_t timeout_us, dcr_stream_header* out);

/* Partial retry (sender side).  After a failure the receiver reads back the
 * applied flags of a DELTA stream; this call writes a RETRY stream (as
 * dcr_encode with DCR_MODE_RETRY would) restricted to the chunks that hold at
 * least one record of that stream whose flag is 0, so only the partitions
 * that did not finish are sent again (ai-feeds summary, "key modules" 4).
 * A chunk whose records were all applied is left out; one that was not
 * reached, or was torn by the failure, is sent whole.  The flags must be the
 * ones the receiver's dcr_apply set (a flag is set only after all writes of
 * its record); dcr_apply_overwrite_retry applies the result.
 *   delta_header     the DELTA stream's header, in HOST memory (magic,
 *                    format, chunk size and plan fingerprint are checked:
 *                    DCR_E_FORMAT; stream_kind must be DCR_MODE_DELTA)
 *   delta_dir_dev, delta_dir_bytes  its directory in device memory and the
 *                    buffer's size (at least n_records * 32: DCR_E_INVAL)
 *   delta_flags_dev  one byte per record of that stream, device memory
 *   the remaining arguments as for dcr_encode (the workspace needs no more).
 * Only the listed chunks are read from the shards.  A directory entry that
 * names no chunk of the plan makes result->status DCR_E_FORMAT (no usable
 * stream). */
int32_t dcr_encode_retry_partial(const dcr_plan* plan,
                                 const void* const* old_shards, const void* const* new_shards,
                                 const dcr_stream_header* delta_header,
                                 const void* delta_dir_dev, uint64_t delta_dir_bytes,
                                 const uint8_t* delta_flags_dev,
                                 uint64_t base_version, uint64_t new_version,
                                 void* header_dev, void* dir_dev, uint64_t dir_cap,
                                 void* payload_dev, uint64_t payload_cap,
                                 dcr_encode_result* result_dev,
                                 void* workspace_dev, uint64_t ws_bytes, void* stream);

/* RETRY stream from a DELTA stream (sender side).  The overwrite retry
 * re-sends every changed element with its new bits (tokendh blog, "no backup
 * copy"; ai.info abstract).  The DELTA stream of the same
 * refit step names every changed element with its XOR mask or its new bits,
 * so this call writes the stream dcr_encode with DCR_MODE_RETRY would write
 * (the same bytes, the same header versions as the DELTA stream's) while
 * reading only the DELTA stream and old at the changed elements; the new
 * shards are not read.  It pays off at low change rates (about half the
 * time of the RETRY encode at 1 % of BF16 elements changed); on dense
 * chunks, where each thread walks many changes, the encode is faster.
 *   old_shards       the plan's old shards (device; as for dcr_encode)
 *   delta_header     the DELTA stream's header, in HOST memory (magic,
 *                    format, chunk size, plan fingerprint and stream_kind
 *                    DCR_MODE_DELTA are checked: DCR_E_FORMAT)
 *   delta_dir_dev, delta_dir_bytes          its directory (device) and the
 *                    buffer's size (at least n_records * 32: DCR_E_INVAL)
 *   delta_payload_dev, delta_payload_bytes  its payload (device) and the
 *                    buffer's size (at least payload_bytes: DCR_E_INVAL)
 *   options          0, or DCR_ENC_INDEX_LISTS for the index-list layout
 *   the remaining arguments as for dcr_encode (the workspace needs
 *   workspace_bytes; no staging area is used).
 * Every directory entry is checked (tensor, chunk, sizes, order, at most an
 * XOR then an overwrite record per chunk) and every record's change set
 * (bounds, popcounts, disjoint records); a malformed DELTA stream makes
 * result->status DCR_E_FORMAT, and the output buffers then hold no usable
 * stream (a bad entry stops the call before any record is written; a bad
 * change set is found per record, while others are written).  The
 * directory buffer also carries per-record scratch during the call, each
 * slot replaced by its entry.  A stream that does not fit dir_cap /
 * payload_cap gives DCR_E_CAPACITY with its sizes in the result, as
 * dcr_encode does.  Like every call, one workspace serves one call at a
 * time. */
int32_t dcr_encode_retry_from_delta(const dcr_plan* plan, const void* const* old_shards,
                                    const dcr_stream_header* delta_header,
                                    const void* delta_dir_dev, uint64_t delta_dir_bytes,
                                    const void* delta_payload_dev, uint64_t delta_payload_bytes,
                                    uint32_t options,
                                    void* header_dev, void* dir_dev, uint64_t dir_cap,
                                    void* payload_dev, uint64_t payload_cap,
                                    dcr_encode_result* result_dev,
                                    void* workspace_dev, uint64_t ws_bytes, void* stream);

/* Apply records [first_record, first_record + n_records) of a stream in place
 * (receiver side).
 * Passages: the receiver XORs each mask into its existing parameter buffer and
 * writes overwrite records in place, and the stream is bound to the base
 * version it was computed from (ai-feeds summary "key modules" 4); a XOR
 * applied twice undoes itself, so each record carries a unique id and is
 * applied once (tokendh blog "XOR or overwrite"); new = old ^ mask
 * (humansand "weight teleportation" page, "Delta update algebra").
 *   canon          host array of n_tensors device pointers, one per canonical
 *                  tensor (numel * elem_bytes bytes, 16-byte aligned)
 *   header         the stream header, in HOST memory; its magic, format, chunk
 *                  size and plan fingerprint must match (DCR_E_FORMAT) and its
 *                  base_version must equal expected_base_version (DCR_E_VERSION)
 *   dir_dev, payload_dev  the stream's directory and payload in device memory
 *   applied_flags_dev     one byte per record of the stream, zeroed by the
 *                  caller once per stream: a record whose flag is set is
 *                  skipped, an applied record gets its flag set (dedup)
 * Each record is checked on the device before it is touched (tensor, chunk,
 * sizes, modes, bounds, bitmap popcount); a malformed record is refused,
 * counted in result_dev and leaves memory untouched.  XOR and overwrite
 * records of one chunk must not mark elements of the same 16-byte group. */
int32_t dcr_apply(const dcr_plan* plan, void* const* canon,
                  const dcr_stream_header* header,
                  const void* dir_dev, const void* payload_dev,
                  uint8_t* applied_flags_dev,
                  uint64_t first_record, uint64_t n_records,
                  uint64_t expected_base_version,
                  dcr_apply_result* result_dev,
                  void* workspace_dev, uint64_t ws_bytes, void* stream);

/* Re-apply every record of a RETRY stream (header stream_kind must be
 * DCR_MODE_RETRY, every record an overwrite) as an overwrite, ignoring and
 * not touching dedup flags.
 * Passages: after a failure the whole change set is re-sent as overwrites,
 * which are idempotent, so no backup copy is kept (tokendh blog "no backup
 * copy"); receivers end with the same bits a dense refit gives and recover
 * fully from failures during the refit (ai.info abstract).  Overwrites are idempotent, so any partial, torn
 * or duplicated earlier apply ends at the new bits. */
int32_t dcr_apply_overwrite_retry(const dcr_plan* plan, void* const* canon,
                                  const dcr_stream_header* header,
                                  const void* dir_dev, const void* payload_dev,
                                  uint64_t expected_base_version,
                                  dcr_apply_result* result_dev,
                                  void* workspace_dev, uint64_t ws_bytes, void* stream);

/* Apply into a receiver's own layout (receiver side).  The receiver stores the
 * canonical tensors in shards of its own (its engine's sharding, interleaved
 * or transposed storage), described by a plan built from its segments over
 * the same tensor table, so the stream's plan fingerprint matches.  The
 * records are written straight into those shards through the receiver plan's
 * pieces; elements of a shard that no segment covers are never touched.
 * The native loader then needs no reload (ai-feeds summary "key modules" 4:
 * the receiver applies the delta to its local checkpoint storage).
 *   plan          the RECEIVER plan (uploaded); DCR_E_INVAL if it maps two
 *                 canonical elements to one shard element
 *   shards        host array of its n_shards device pointers (16-byte
 *                 aligned; NULL only for empty shards)
 *   the remaining arguments as for dcr_apply.  Chunks whose 16-byte groups
 *   sit inside one aligned piece get 128-bit read-modify-writes; the others
 *   are updated element by element. */
int32_t dcr_apply_sharded(const dcr_plan* plan, void* const* shards,
                          const dcr_stream_header* header,
                          const void* dir_dev, const void* payload_dev,
                          uint8_t* applied_flags_dev,
                          uint64_t first_record, uint64_t n_records,
                          uint64_t expected_base_version,
                          dcr_apply_result* result_dev,
                          void* workspace_dev, uint64_t ws_bytes, void* stream);

/* dcr_apply_overwrite_retry into a receiver's own layout, as dcr_apply_sharded. */
int32_t dcr_apply_overwrite_retry_sharded(const dcr_plan* plan, void* const* shards,
                                          const dcr_stream_header* header,
                                          const void* dir_dev, const void* payload_dev,
                                          uint64_t expected_base_version,
                                          dcr_apply_result* result_dev,
                                          void* workspace_dev, uint64_t ws_bytes, void* stream);

/* Transport packing (sender side, after the encode): the pages compress the
 * sparse mask stream before it travels (ai-feeds summary "key modules" 3;
 * humansand "weight teleportation" page, "A strong baseline with
 * Blackwell-native DE", on codecs for masks that are mostly runs of zeros).
 * Every index-list record (DCR_ENC_INDEX_LISTS) whose list, written as gap
 * varints, takes strictly fewer padded bytes gets its first section
 * replaced: change j's gap is its index minus the previous change's index
 * minus one (change 0's gap is its index), each gap an unsigned LEB128
 * varint (seven bits per byte, low group first, the high bit set on every
 * byte but the last), the varints back to back, zero-padded to 16 bytes;
 * its entry gets layout DCR_LAYOUT_GAPS and its new offset and size.  Every
 * other record is copied unchanged.  The output header is the input's with
 * magic DCR_MAGIC_PACKED and the packed payload size.  A packed stream is a
 * transport form only: dcr_apply refuses it; dcr_stream_unpack turns it
 * back into the stream it was made from, byte for byte.
 *   header         the input stream's header in HOST memory: a plain stream
 *                  (DCR_MAGIC) of this plan (fingerprint), at most two
 *                  records per chunk; else DCR_E_FORMAT
 *   dir_dev, payload_dev            the input stream (device)
 *   header_out_dev, dir_out_dev, dir_cap, payload_out_dev, payload_cap
 *                  the output stream (device); dir_cap of at least
 *                  n_records * 32 bytes (DCR_E_CAPACITY otherwise, before
 *                  any launch): the output directory also carries
 *                  per-record scratch during the call
 *   result_dev     n_records, payload_bytes (the output's size, also when it
 *                  did not fit) and status: DCR_OK; DCR_E_CAPACITY when
 *                  payload_cap is smaller; DCR_E_FORMAT when an entry does
 *                  not describe a record of the format inside the payload,
 *                  or a list is not strictly ascending below its chunk's
 *                  elements (the outputs then hold no usable stream)
 *   workspace_dev, ws_bytes         at least the plan's workspace_bytes */
int32_t dcr_stream_pack(const dcr_plan* plan, const dcr_stream_header* header,
                        const void* dir_dev, const void* payload_dev,
                        void* header_out_dev, void* dir_out_dev, uint64_t dir_cap,
                        void* payload_out_dev, uint64_t payload_cap,
                        dcr_encode_result* result_dev,
                        void* workspace_dev, uint64_t ws_bytes, void* stream);

/* The inverse of dcr_stream_pack (receiver side, before the apply): gap
 * records back to index lists, every other record copied, header magic back
 * to DCR_MAGIC.  Arguments as for dcr_stream_pack, with a packed stream's
 * header (DCR_MAGIC_PACKED).  result->status DCR_E_FORMAT: an entry that does
 * not describe a record inside the payload or does not start where the
 * previous one ends; a gap section that is not exactly K minimal varints
 * (at most three bytes, values below 2^16) followed by zero bytes, or a
 * last index at or past its chunk's elements. */
int32_t dcr_stream_unpack(const dcr_plan* plan, const dcr_stream_header* header,
                          const void* dir_dev, const void* payload_dev,
                          void* header_out_dev, void* dir_out_dev, uint64_t dir_cap,
                          void* payload_out_dev, uint64_t payload_cap,
                          dcr_encode_result* result_dev,
                          void* workspace_dev, uint64_t ws_bytes, void* stream);

/* Benchmark hook.  While set (both non-NULL), every encode, apply or retry
 * call made on this host thread records `start` on its stream just before its
 * main kernel (the encode tile kernels, or the apply kernel) and `stop` just
 * after it, so that hipEventElapsedTime gives that kernel's duration alone.
 * The events are hipEvent_t handles the caller created; NULL, NULL turns the
 * hook off.  An encode that runs in slices (dcr_encode_pipelined) has no
 * single main kernel and records neither event; with a compact staging area
 * the chunks encoded again after the fix-up are outside the events.  Never
 * fails. */
void dcr_set_kernel_events(void* start, void* stop);

/* Message of the last error on this thread ("" if none). */
const char* dcr_last_error(void);

/* Format constants as this library defines them, for cross-checks:
 * out[0..9] = magic, format version, chunk bytes, header bytes, dirent bytes,
 * sizeof(dcr_tensor_desc), sizeof(dcr_segment), sizeof(dcr_stream_header),
 * DCR_ENC_INDEX_LISTS, DCR_LAYOUT_LIST.
 * Returns the number written (at most n). */
uint32_t dcr_format_constants(uint32_t* out, uint32_t n);

#ifdef __cplusplus
}
#endif
#endif /* DCR_H */
