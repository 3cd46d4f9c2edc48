/*
 * dcr_oracle.h -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, single-threaded CPU definition of bit-exact delta-compressed refit
 * (encode / apply / overwrite-retry) on host memory.  It exists to check the
 * GPU library against; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load it.  It shares no source, header, table
 * or constant with the GPU library: every format constant below is defined
 * here independently, and a test checks that both sides agree.
 *
 * Method sources (pages on NeMo-DCR, "bit-exact delta-compressed refit"):
 *   - change detection on stored bits, per owned training shard:
 *     ai-feeds summary, "Method / input and change detection"; tokendh blog,
 *     "shard owner" section (compare bit patterns, not float values, so +0/-0
 *     differ).
 *   - direct projection (fixed affine map shard index -> canonical checkpoint
 *     coordinate) and residual conversion (re-assemble canonical fragment, diff,
 *     emit overwrite records): ai-feeds summary, "key modules" 1 and 2;
 *     ai.info abstract.
 *   - XOR masks for affine changes, overwrite for the rest, one delta stream:
 *     ai-feeds summary, "key modules" 2-3; tokendh blog, "XOR or overwrite".
 *   - in-place apply, dedup by unique ids, whole-set overwrite retry, version
 *     binding: ai-feeds summary, "key modules" 4; tokendh blog, "XOR or
 *     overwrite" (dedup) and "no backup copy" (retry, joint commit).
 *   - delta algebra mask = old XOR new, new = old XOR mask on a flat bit
 *     buffer: humansand "weight teleportation" page, "Delta update algebra".
 * The pages fix no record layout; the chunked byte-plane record format used
 * here (64 KiB canonical chunks, change bitmap, byte planes, elided zero high
 * bytes) is this project's own and is written out in the design notes.
 */
#ifndef DCR_ORACLE_H
#define DCR_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define ORC_OK          0
#define ORC_E_INVAL    -1
#define ORC_E_COVERAGE -2
#define ORC_E_FORMAT   -3
#define ORC_E_VERSION  -4
#define ORC_E_CAPACITY -5
#define ORC_E_NOMEM    -7

/* routes */
#define ORC_ROUTE_AFFINE_XOR   0
#define ORC_ROUTE_OVERWRITE    1
#define ORC_ROUTE_BLOCK_SCALED 2

/* stream kinds / encode modes */
#define ORC_MODE_DELTA 0
#define ORC_MODE_RETRY 1

/* encode option (OR-ed into the mode): low-density records carry a list of
 * 16-bit element indices instead of the change bitmap when that list is
 * strictly smaller (next-step variant; the pages compress the mask stream,
 * ai-feeds summary "key modules" 3) */
#define ORC_ENC_LISTS 0x100u

/* record layouts (directory entry byte 15) */
#define ORC_LAYOUT_BITMAP 0
#define ORC_LAYOUT_LIST   1

/* record kinds, high-byte modes */
#define ORC_KIND_XOR 0
#define ORC_KIND_OW  1
#define ORC_HI_NONE   0
#define ORC_HI_SPARSE 1
#define ORC_HI_DENSE  2

#define ORC_MAGIC       0x31524344u /* "DCR1" little-endian */
#define ORC_FORMAT_VER  1u
#define ORC_CHUNK_BYTES 65536u
#define ORC_HEADER_BYTES 64u
#define ORC_DIRENT_BYTES 32u

/* One canonical tensor.  24 bytes. */
typedef struct {
    uint64_t numel;
    uint32_t elem_bytes;   /* 1, 2 or 4 */
    uint32_t route;        /* ORC_ROUTE_* */
    int32_t  scale_tensor; /* BLOCK_SCALED: id of its fp32 scale tensor, else -1 */
    uint32_t scale_block;  /* BLOCK_SCALED: elements per scale */
} orc_tensor;

/* One affine segment: for every multi-index x in [0, extent),
 * canonical element canon_off + sum_d x_d*canon_stride_d of tensor tensor_id
 * is stored at element shard_off + sum_d x_d*shard_stride_d of shard shard_id
 * (element units of the tensor's width).  128 bytes. */
typedef struct {
    uint32_t tensor_id, shard_id, ndim, reserved;
    uint64_t shard_off, canon_off;
    uint64_t extent[4];
    int64_t  shard_stride[4];
    int64_t  canon_stride[4];
} orc_segment;

/* FNV-1a-64 over the serialised tensor table. */
uint64_t orc_fingerprint(const orc_tensor* T, uint32_t nT);

/* Encode.  Writes the 64-byte header, the directory and the payload into the
 * caller's buffers.  *dir_bytes / *payload_bytes receive the required sizes
 * even when the call fails with ORC_E_CAPACITY (then nothing usable is
 * written). */
int32_t orc_encode(const orc_tensor* T, uint32_t nT,
                   const void* const* old_shards, const void* const* new_shards,
                   const uint64_t* shard_bytes, uint32_t nS,
                   const orc_segment* segs, uint64_t nseg,
                   uint32_t mode, uint64_t base_version, uint64_t new_version,
                   uint8_t* header_out,
                   uint8_t* dir_out, uint64_t dir_cap, uint64_t* dir_bytes,
                   uint8_t* payload_out, uint64_t payload_cap, uint64_t* payload_bytes);

/* Partial retry (ai-feeds summary, "key modules" 4: after a failure only the
 * partitions that did not finish are sent again): a RETRY stream, as
 * orc_encode with ORC_MODE_RETRY would write it, restricted to the chunks that
 * hold at least one record of the DELTA stream (delta_header, delta_dir)
 * whose applied flag (delta_flags, one byte per record) is 0.  A chunk the
 * receiver finished is left out; one it did not finish, or tore, is sent
 * whole.  ORC_E_FORMAT if the header is not a DELTA stream of this tensor
 * table or an entry names no chunk of it. */
int32_t orc_encode_retry_partial(const orc_tensor* T, uint32_t nT,
                                 const void* const* old_shards, const void* const* new_shards,
                                 const uint64_t* shard_bytes, uint32_t nS,
                                 const orc_segment* segs, uint64_t nseg,
                                 const uint8_t* delta_header, const uint8_t* delta_dir,
                                 const uint8_t* delta_flags,
                                 uint64_t base_version, uint64_t new_version,
                                 uint8_t* header_out,
                                 uint8_t* dir_out, uint64_t dir_cap, uint64_t* dir_bytes,
                                 uint8_t* payload_out, uint64_t payload_cap, uint64_t* payload_bytes);

/* Materialise canonical tensor t from shards (the direct projection alone). */
int32_t orc_gather(const orc_tensor* T, uint32_t nT,
                   const void* const* shards, const uint64_t* shard_bytes, uint32_t nS,
                   const orc_segment* segs, uint64_t nseg,
                   uint32_t t, void* out);

/* Validate a whole stream against the tensor table (header, directory,
 * every record's bytes).  ORC_OK or ORC_E_FORMAT / ORC_E_VERSION. */
int32_t orc_validate(const orc_tensor* T, uint32_t nT, const uint8_t* header,
                     const uint8_t* dir, const uint8_t* payload,
                     uint64_t expected_base_version, int32_t require_kind);

/* Apply records [first, first+n) of a stream in place to canonical tensors
 * canon[t] (host memory, numel*elem_bytes bytes each).  Records whose flag is
 * set are skipped; applied records get their flag set.  The stream is
 * validated as a whole before anything is written. */
int32_t orc_apply(const orc_tensor* T, uint32_t nT, void* const* canon,
                  const uint8_t* header, const uint8_t* dir, const uint8_t* payload,
                  uint8_t* flags, uint64_t first, uint64_t n,
                  uint64_t expected_base_version);

/* Apply every record of a RETRY stream as an overwrite, ignoring flags. */
int32_t orc_apply_overwrite_retry(const orc_tensor* T, uint32_t nT, void* const* canon,
                                  const uint8_t* header, const uint8_t* dir,
                                  const uint8_t* payload, uint64_t expected_base_version);

/* Transport packing of a stream (the pages compress the sparse mask stream
 * before it travels: ai-feeds summary, "key modules" 3; humansand "weight
 * teleportation" page, "A strong baseline with Blackwell-native DE", on
 * codecs for masks that are mostly runs of zeros).  Every index-list record
 * whose list takes fewer padded bytes as gap varints gets its first section
 * replaced: change j's index i_j becomes the gap g_0 = i_0, g_j = i_j - i_{j-1} - 1,
 * each written as an unsigned LEB128 varint (seven bits per byte, low
 * group first, high bit set on every byte but the last), the K varints
 * back to back and zero-padded to 16 bytes; its directory entry gets
 * layout ORC_LAYOUT_GAPS.  Other records are copied unchanged.  Offsets
 * are recomputed; the header's magic becomes ORC_MAGIC_PACKED and its
 * payload_bytes the packed total.  The input must validate (ORC_E_FORMAT /
 * ORC_E_VERSION otherwise); *payload_bytes gets the packed size, and
 * ORC_E_CAPACITY if payload_cap is smaller (nothing usable written). */
#define ORC_LAYOUT_GAPS  2
#define ORC_MAGIC_PACKED 0x50524344u /* "DCRP" little-endian */
int32_t orc_stream_pack(const orc_tensor* T, uint32_t nT, const uint8_t* header,
                        const uint8_t* dir, const uint8_t* payload,
                        uint8_t* header_out, uint8_t* dir_out,
                        uint8_t* payload_out, uint64_t payload_cap, uint64_t* payload_bytes);

/* The inverse: a packed stream back to the stream it was packed from.
 * Refused (ORC_E_FORMAT): a header that is not a packed stream of this
 * tensor table; a gap section that does not hold exactly K minimal varints
 * (a longer encoding of a value, a value that does not fit 16 bits, a
 * varint cut off by the section's end) followed by zero bytes; an index at
 * or past the chunk's elements; any record of the output that does not
 * validate. */
int32_t orc_stream_unpack(const orc_tensor* T, uint32_t nT, const uint8_t* header,
                          const uint8_t* dir, const uint8_t* payload,
                          uint8_t* header_out, uint8_t* dir_out,
                          uint8_t* payload_out, uint64_t payload_cap, uint64_t* payload_bytes);

/* Apply only elements [elem_lo, elem_hi) of one record (a torn write); no flag. */
int32_t orc_apply_record_part(const orc_tensor* T, uint32_t nT, void* const* canon,
                              const uint8_t* dir, const uint8_t* payload,
                              uint64_t rec, uint32_t change_lo, uint32_t change_hi);

#ifdef __cplusplus
}
#endif
#endif
