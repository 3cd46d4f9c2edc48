// dcr_internal.h -- plan layout shared by the host plan builder and the
// gfx950 kernels of libdcr.so.  Not part of the public ABI.
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

#include "dcr.h"

namespace dcr {

constexpr uint32_t kChunkBytes = DCR_CHUNK_BYTES;   // canonical bytes per chunk
constexpr uint32_t kVecBytes = 16;                  // one 128-bit access
constexpr uint32_t kVecsPerChunk = kChunkBytes / kVecBytes;  // 4096
constexpr uint32_t kThreads = 1024;                 // workgroup of encode / apply
constexpr uint32_t kVecsPerThread = kVecsPerChunk / kThreads;  // 4
constexpr uint32_t kMaxCachedPieces = 64;           // pieces of a chunk kept in LDS
constexpr uint32_t kWinBytes = 12288;               // LDS output window of the encode record writer
// largest payload of one chunk's records (mixed XOR + OW on BF16: two 4 KiB
// bitmaps + 2 bytes per change + padding), rounded up to 16
constexpr uint32_t kStageBytes = 73792;

// status word of the decoupled look-back: 2 flag bits, then a packed value
// (records << 36 | payload_bytes / 16)
constexpr uint64_t kFlagAgg = 1, kFlagIncl = 2;
constexpr int kValShift = 2;
constexpr int kRecShift = 36;
constexpr uint64_t kP16Mask = (uint64_t(1) << kRecShift) - 1;
// tiles (chunks) of a plan: the encode launches one kThreads workgroup per
// tile in one grid, whose work-items must fit 32 bits (4 194 303 chunks,
// 256 GiB of canonical BF16); this also keeps 2 records per tile below 2^26
constexpr uint64_t kMaxTiles = uint64_t(0xFFFFFFFFu) / kThreads;
constexpr uint32_t kFixTiles = 256;                 // tiles per workgroup of the encode fix-up
// encode counters (uint32 words at ws_counter): [0] tile claim, [1] fix-up
// block claim, [2..3] changed elements, [4..5] stream total
// (records << 36 | payload / 16)
constexpr uint32_t kCtrTile = 0, kCtrFix = 1, kCtrChanged = 2, kCtrTotal = 4;
// apply counters (uint32 words at ws_counter): [8] records deferred to the
// large-record kernel
constexpr uint32_t kCtrBig = 8;
// partial retry: [10] nonzero if a DELTA directory entry named no chunk
constexpr uint32_t kCtrBad = 10;
// The counter area is kCtrBytes long: the uint32 counters above in its first
// 256 bytes, then the staging claim counters (kStageParts uint64, one per
// partition of the staging area, at byte kStageCtrOff), then the count of
// tiles to encode again (uint32 at byte kRedoCtrOff).  All zeroed per encode.
constexpr uint32_t kCtrBytes = 1024, kStageParts = 64, kStageCtrOff = 256, kRedoCtrOff = 768;
// a tile whose records found no room in a compact staging area
constexpr uint64_t kNoClaim = ~uint64_t(0);
constexpr uint32_t kSmallThreads = 256;             // workgroup of the small-record apply
constexpr uint32_t kSmallStage = 16384;             // its LDS stage (records up to this size)
// the small-record apply reads and writes whole 128-byte lines for records
// whose changes are at least 1/kLineDensity of their chunk's elements
constexpr uint32_t kLineDensity = 80;

// Device-side tensor descriptor.  48 bytes.
struct DevTensor {
    uint64_t numel;
    uint64_t scale_bit_off;    // BLOCK_SCALED: bit offset of its scale tensor's flags
    uint32_t w;
    uint32_t route;
    uint32_t n_chunks;
    int32_t scale_tensor;
    uint32_t scale_block;
    uint32_t first_chunk;      // plan index of chunk 0
    uint32_t pad[2];
};
static_assert(sizeof(DevTensor) == 48, "DevTensor");

// One canonical chunk (one encode tile).  16 bytes.  n_pieces carries flags
// in its top byte (kChunkDirect).
struct DevChunk {
    uint32_t tensor;
    uint32_t chunk_idx;
    uint32_t first_piece;
    uint32_t n_pieces;
};
constexpr uint32_t kPiecesMask = 0xFFFFFFu;
// every 16-byte group of the chunk lies inside one piece at a 16-byte aligned
// shard offset, and the chunk has at most kMaxCachedPieces pieces
constexpr uint32_t kChunkDirect = 1u << 24;
static_assert(sizeof(DevChunk) == 16, "DevChunk");

// A contiguous run of a chunk: canonical elements [canon_start, canon_start+len)
// of the chunk are shard elements [shard_elem_off, +len) of shard `shard`.  16 bytes.
struct DevPiece {
    uint64_t shard_elem_off;
    uint32_t shard;
    uint16_t canon_start;      // first canonical element of the run within the chunk
    uint16_t len_m1;           // run length - 1 (lengths 1 .. 65536)
};
static_assert(sizeof(DevPiece) == 16, "DevPiece");

struct Plan {
    std::vector<dcr_tensor_desc> tensors;
    std::vector<uint64_t> shard_bytes;
    std::vector<DevTensor> dt;
    std::vector<DevChunk> chunks;
    std::vector<DevPiece> pieces;
    std::vector<uint32_t> scale_chunks;   // chunks of scale tensors that gate a BLOCK_SCALED one
    std::vector<uint64_t> slots;          // per chunk: staging slot offset (prefix of worst cases)
    std::vector<uint32_t> slow;           // chunks without kChunkDirect
    std::vector<uint32_t> direct[3];      // direct chunks of 1-, 2-, 4-byte elements
    uint64_t fingerprint = 0;
    uint64_t canonical_bytes = 0;
    bool shard_disjoint = true;           // no shard element holds two canonical elements
    uint64_t scale_bits = 0;              // total flag bits (multiple of 64)
    uint64_t max_dir_bytes = 0, max_payload_bytes = 0;
    uint64_t compact_stage_bytes = 0;     // least staging area used compactly
    // device table layout
    uint64_t off_tensors = 0, off_chunks = 0, off_pieces = 0, off_scale_chunks = 0, off_slots = 0, off_slow = 0,
             off_direct[3] = {0, 0, 0}, table_bytes = 0;
    // workspace layout
    uint64_t ws_status = 0, ws_fix = 0, ws_need = 0, ws_counter = 0, ws_old = 0, ws_new = 0, ws_scale = 0, ws_canon = 0,
             ws_agg = 0, ws_info = 0, ws_big = 0, big_cap = 0, ws_soff = 0, ws_bytes = 0;
    std::vector<uint8_t> blob;            // host image of the device tables
    void* dev_tables = nullptr;           // bound by dcr_plan_upload
    uint32_t widths = 0;                  // the element widths of the chunks, OR-ed (1 | 2 | 4)
};

void set_error(const std::string& msg);

}  // namespace dcr

struct dcr_plan : dcr::Plan {};
