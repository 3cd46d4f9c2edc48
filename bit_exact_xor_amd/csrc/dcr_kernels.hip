// dcr_kernels.hip -- gfx950 kernels and device-side entry points of libdcr.so.
//
// encode (sender): one workgroup of 1024 threads per 64 KiB canonical chunk
//   ("tile").  It gathers the chunk's old and new bytes from the trainer
//   shards through the plan's pieces (the direct projection: ai-feeds summary
//   "key modules" 1), 16 bytes per lane per load.  It compares stored bits as
//   integers (tokendh blog "shard owner": +0/-0 differ) and routes each
//   16-byte group to XOR or overwrite (ai-feeds "key modules" 2-3).  Change
//   counts are scanned per workgroup and the records are assembled in LDS and
//   written with 128-bit stores.  With a staging area holding a slot for
//   every chunk (the default), each tile writes its records to its slot and
//   publishes its record count and payload size; a fix-up pass scans those
//   sizes (a decoupled look-back across fix-up blocks of 256 tiles) into
//   directory indices and payload offsets and moves the records into place.
//   With a smaller area, tiles claim exact bytes in partitions of it, and
//   chunks that find no room are encoded again after the fix-up.  Without
//   one, each tile finds its offsets by a decoupled look-back over all
//   earlier tiles, begun once its first record window is assembled, and
//   writes in place; that kernel is built once per set of element widths.
// apply (receiver): one workgroup per directory entry.  It checks the entry
//   and the record bytes before touching anything, stages the record in LDS,
//   ranks the changes by a workgroup scan of the bitmap, and updates every
//   touched 16-byte group of the canonical tensor with one 128-bit
//   read-modify-write: XOR for masks, assignment for overwrites (ai-feeds
//   "key modules" 4; humansand "Delta update algebra").  Dense records read
//   and write their touched 128-byte lines whole, and a chunk's XOR record
//   applies the overwrite record next to it in the same pass.  Dedup flags
//   make a duplicate a no-op (tokendh "XOR or overwrite"); the retry ignores
//   them and overwrites (tokendh "no backup copy").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstring>
#include <mutex>
#include <thread>
#include <string>

#include "dcr_internal.h"

namespace dcr {

// ------------------------------------------------------------ device helpers

__device__ __forceinline__ uint32_t dpad16(uint32_t x) { return (x + 15u) & ~15u; }

// The thread index, opaque to the compiler: values derived from it are
// recomputed where they are used instead of being kept live in registers.
__device__ __forceinline__ uint32_t opaque_tid() {
    uint32_t t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}
__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }

__device__ __forceinline__ uint64_t ld_status(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_status(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t wave_incl_scan(uint64_t x, uint32_t lane) {
#pragma unroll
    for (uint32_t d = 1; d < 64; d <<= 1) {
        uint64_t y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    return x;
}

__device__ __forceinline__ uint64_t wave_sum(uint64_t x) {
#pragma unroll
    for (uint32_t d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
    return x;
}

// Inclusive wave64 scan of a 32-bit value by DPP lane moves (no LDS): the
// three preceding lanes' original values within each row of 16, then the
// partial sums 4 and 8 lanes back (banks past the first), then the last lane
// of row 0 broadcast into rows 1 and 3 and the last lane of row 1 into rows
// 2 and 3.  Lanes a move leaves out add nothing.
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t x) {
    const uint32_t x0 = x;
    x += __builtin_amdgcn_update_dpp(0u, x0, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0u, x0, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0u, x0, 0x113, 0xf, 0xf, true);   // row_shr:3
    x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xe, false);   // row_shr:4, banks 1-3
    x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xc, false);   // row_shr:8, banks 2-3
    x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);   // row_bcast:15, rows 1 and 3
    x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);   // row_bcast:31, rows 2 and 3
    return x;
}

// The same over a 64-bit value whose two 32-bit halves never carry into each
// other: packed 16-bit counts whose workgroup sums stay below 65536, or a
// plain count whose sum stays below 2^32.
__device__ __forceinline__ uint64_t wave_incl_scan_halves(uint64_t x) {
    return uint64_t(wave_incl_scan_dpp(uint32_t(x))) | (uint64_t(wave_incl_scan_dpp(uint32_t(x >> 32))) << 32);
}

// Exclusive workgroup scan of N packed 64-bit values; totals returned in tot.
// Each value's halves are scanned apart (wave_incl_scan_halves), so every
// caller's values keep their sums inside each 32-bit half.  Uses
// sh[2 * N * 16 + N] of LDS; ends with a barrier so sh may be reused.  The
// first wave scans the 16 wave totals, so that each thread reads back just
// two values per scanned quantity.
template <int N>
__device__ __forceinline__ void block_excl_scan(uint64_t (&v)[N], uint64_t (&tot)[N], uint64_t* sh) {
    constexpr uint32_t NW = kThreads / 64;
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    uint64_t inc[N];
#pragma unroll
    for (int i = 0; i < N; i++) inc[i] = wave_incl_scan_halves(v[i]);
    if (lane == 63) {
#pragma unroll
        for (int i = 0; i < N; i++) sh[i * NW + wave] = inc[i];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int i = 0; i < N; i++) {
            const uint64_t t = lane < NW ? sh[i * NW + lane] : 0;
            const uint64_t ti = wave_incl_scan_halves(t);
            if (lane < NW) sh[N * NW + i * NW + lane] = ti - t;      // exclusive wave prefix
            if (lane == NW - 1) sh[2 * N * NW + i] = ti;            // total
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; i++) {
        v[i] = sh[N * NW + i * NW + wave] + inc[i] - v[i];
        tot[i] = sh[2 * N * NW + i];
    }
    __syncthreads();
}

__device__ __forceinline__ uint32_t field16(uint64_t packed, int k) {
    return uint32_t(packed >> (16 * k)) & 0xFFFFu;
}

// Element e (a compile-time index after unrolling) of a 16-byte group of
// W-byte elements held in 4 registers.
template <int W>
__device__ __forceinline__ uint32_t elem(const uint32_t (&q)[4], uint32_t e) {
    if constexpr (W == 4) return q[e];
    else if constexpr (W == 2) return (q[e >> 1] >> (16u * (e & 1u))) & 0xFFFFu;
    else return (q[e >> 2] >> (8u * (e & 3u))) & 0xFFu;
}
// OR v into element e (compile-time index; the element's bits must be zero).
template <int W>
__device__ __forceinline__ void set_elem(uint32_t (&q)[4], uint32_t e, uint32_t v) {
    if constexpr (W == 4) q[e] |= v;
    else if constexpr (W == 2) q[e >> 1] |= (v & 0xFFFFu) << (16u * (e & 1u));
    else q[e >> 2] |= (v & 0xFFu) << (8u * (e & 3u));
}
__device__ __forceinline__ uint32_t sgpr(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
// A workgroup-uniform struct loaded from memory, moved word by word into
// scalar registers (the loads themselves cannot be scalar once the kernel has
// written memory, and vector copies would occupy VGPRs for the whole tile).
template <typename T>
__device__ __forceinline__ T uniform_load(const T* p) {
    static_assert(sizeof(T) % 4 == 0, "uniform_load");
    const T v = *p;
    uint32_t w[sizeof(T) / 4];
    __builtin_memcpy(w, &v, sizeof(T));
#pragma unroll
    for (uint32_t i = 0; i < sizeof(T) / 4; i++) w[i] = __builtin_amdgcn_readfirstlane(w[i]);
    T r;
    __builtin_memcpy(&r, w, sizeof(T));
    return r;
}
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) v4u* gv4p;   // global (not flat) 128-bit loads

// chunk element -> index of the piece holding it (largest start <= e)
__device__ __forceinline__ uint32_t find_piece(const DevPiece* pc, uint32_t n, uint32_t e) {
    uint32_t lo = 0, hi = n;  // invariant: pc[lo].canon_start <= e
    while (hi - lo > 1) {
        uint32_t mid = (lo + hi) >> 1;
        if (pc[mid].canon_start <= e) lo = mid;
        else hi = mid;
    }
    return lo;
}

// ------------------------------------------------------------------ encode

struct EncodeArgs {
    const DevTensor* tensors;
    const DevChunk* chunks;
    const DevPiece* pieces;
    const uint8_t* const* old_sh;
    const uint8_t* const* new_sh;
    const uint64_t* scale_flags;
    uint64_t* status;
    uint32_t* counter;      // encode counters (kCtr*)
    uint64_t* tile_agg;     // per tile: records << 36 | payload / 16
    uint64_t* tile_info;    // per tile: Kx | Ko << 17 | Hx << 34
    const uint64_t* slots;  // per tile: staging slot offset
    uint8_t* stage;         // staging area (staged launches)
    uint8_t* dir;
    uint8_t* payload;
    uint64_t dir_cap;       // bytes
    uint64_t payload_cap;   // bytes
    const uint64_t* need;   // partial retry: one bit per tile, set = encode it (NULL: every tile)
    uint64_t* soff;         // compact staging: per tile, the staging offset it claimed (or kNoClaim)
    unsigned long long* stage_ctr;   // compact staging: bytes claimed in each of kStageParts partitions
    uint64_t part_bytes;    // compact staging: bytes of one partition
    uint32_t n_tiles;
    uint32_t mode;
    uint32_t lists;         // 1: index-list layout allowed for low-density records
    uint32_t compact;       // 1: tiles claim exactly their records' bytes of the staging area
};

struct EncodeShared {
    alignas(16) uint32_t pw[kVecsPerChunk][4];   // payload words of changed groups
    alignas(16) uint8_t win[kWinBytes];         // output window of the record writer
    DevPiece pieces[kMaxCachedPieces];
    uint32_t pstart[kMaxCachedPieces];      // first chunk element of each piece
    uint32_t pend[kMaxCachedPieces];        // one past its last
    uint64_t pold[kMaxCachedPieces];        // old / new address of the piece's first element
    uint64_t pnew[kMaxCachedPieces];
    uint64_t scan[2 * 3 * (kThreads / 64) + 3];
    uint64_t excl;
    uint64_t claim;   // compact staging: the claimed offset; in order: the records' address (0: no room)
    uint32_t next;
};

// Sizes and high-byte mode of a chunk's records (the record layout of the
// format): bitmap, low plane, then for 2-byte XOR records a sparse (presence
// bitmap + nonzero high bytes) or dense high plane, whichever is smaller
// (dense on a tie); overwrite records carry all W byte planes.  With index
// lists allowed, a record whose K 16-bit indices (padded) take fewer bytes
// than its padded bitmap carries them in the bitmap's place.
struct RecLayout {
    uint32_t size_x, size_o;     // bytes of the XOR / overwrite record (0: none)
    uint32_t mode_x, h_x;        // XOR record: hi_mode and its H field
    uint32_t off_pres, off_hi_x; // XOR record: presence bitmap / high plane offsets
    uint32_t head_x, head_o;     // bytes of each record's first section (bitmap or index list)
    uint32_t list_x, list_o;     // 1: index-list layout
};

__device__ __forceinline__ RecLayout rec_layout(uint32_t w, uint32_t n_c, uint32_t Kx, uint32_t Ko, uint32_t Hx,
                                                uint32_t lists) {
    RecLayout L{0, 0, DCR_HI_NONE, 0, 0, 0, 0, 0, 0, 0};
    const uint32_t bm = dpad16((n_c + 7) / 8);
    L.list_x = (lists && Kx && dpad16(2 * Kx) < bm) ? 1u : 0u;
    L.list_o = (lists && Ko && dpad16(2 * Ko) < bm) ? 1u : 0u;
    L.head_x = L.list_x ? dpad16(2 * Kx) : bm;
    L.head_o = L.list_o ? dpad16(2 * Ko) : bm;
    if (Kx) {
        L.size_x = L.head_x + dpad16(Kx);
        L.off_hi_x = L.size_x;
        if (w == 2 && Hx) {
            const uint32_t sparse = dpad16((Kx + 7) / 8) + dpad16(Hx);
            if (sparse < dpad16(Kx)) {
                L.mode_x = DCR_HI_SPARSE;
                L.off_pres = L.size_x;
                L.off_hi_x = L.size_x + dpad16((Kx + 7) / 8);
                L.size_x += sparse;
                L.h_x = Hx;
            } else {
                L.mode_x = DCR_HI_DENSE;
                L.size_x += dpad16(Kx);
                L.h_x = Kx;
            }
        }
    }
    if (Ko) L.size_o = L.head_o + w * dpad16(Ko);
    return L;
}

// Directory entry `which` (0 = first record of the tile) of a tile whose
// records start at payload offset P.
__device__ __forceinline__ void put_dirent(uint8_t* dir, uint64_t index, uint32_t which, uint32_t tensor,
                                           uint32_t chunk, uint32_t w, const RecLayout& L, uint32_t Kx,
                                           uint32_t Ko, uint64_t P) {
    const bool x = Kx && which == 0;
    v4u e0, e1;
    e0.x = tensor;
    e0.y = chunk;
    e0.z = x ? Kx : Ko;
    const uint32_t hm = x ? L.mode_x : (w == 1 ? uint32_t(DCR_HI_NONE) : uint32_t(DCR_HI_DENSE));
    const uint32_t layout = x ? L.list_x : L.list_o;
    e0.w = (x ? 0u : 1u) | (hm << 8) | (w << 16) | (layout << 24);
    const uint64_t off = P + (x ? 0u : L.size_x);
    e1.x = uint32_t(off);
    e1.y = uint32_t(off >> 32);
    e1.z = x ? L.size_x : L.size_o;
    e1.w = x ? L.h_x : (w == 1 ? 0u : Ko);
    v4u* de = reinterpret_cast<v4u*>(dir + index * DCR_DIRENT_BYTES);
    de[0] = e0;
    de[1] = e1;
}

// Decoupled look-back, run by one full wave: the exclusive sum of the values
// of entries [0, idx) of `status`.  Waits until each entry it needs holds at
// least an aggregate; every entry below idx belongs to a workgroup that has
// already started (ids are claimed in order), so the wait ends.
__device__ __forceinline__ uint64_t look_back(const uint64_t* status, uint32_t idx, uint32_t lane) {
    uint64_t excl = 0;
    int64_t hi = int64_t(idx) - 1;
    while (hi >= 0) {
        const int64_t i = hi - int64_t(lane);
        const uint64_t st = i >= 0 ? ld_status(status + i) : kFlagIncl;
        const uint32_t flag = uint32_t(st & 3u);
        const uint64_t incl_m = __ballot(flag == kFlagIncl);
        const uint64_t zero_m = __ballot(flag == 0);
        const uint32_t first = incl_m ? uint32_t(__ffsll((unsigned long long)incl_m) - 1) : 64u;
        const uint64_t need = first >= 63 ? ~uint64_t(0) : ((uint64_t(2) << first) - 1);
        if (zero_m & need) {
            __builtin_amdgcn_s_sleep(1);
            continue;
        }
        excl += wave_sum(lane <= first ? (st >> kValShift) : 0);
        if (first < 64) break;
        hi -= 64;
    }
    return excl;
}

// Gather one 16-byte group (elements e0 .. e0+V-1 of the chunk) of old and
// new from the pieces pc[0..np).  Elements at or past n_c read as zero.
template <int W>
__device__ __forceinline__ void gather_group(const EncodeArgs& a, const DevPiece* pc, uint32_t np, uint32_t e0,
                                             uint32_t n_c, v4u& vo, v4u& vn) {
    constexpr uint32_t V = 16 / W;
    vo = v4u{0, 0, 0, 0};
    vn = v4u{0, 0, 0, 0};
    if (e0 >= n_c) return;
    uint32_t p = find_piece(pc, np, e0);
    uint32_t pstart = pc[p].canon_start, pend = pstart + uint32_t(pc[p].len_m1) + 1;
    if (e0 + V <= pend) {
        const uint64_t off = (pc[p].shard_elem_off + (e0 - pstart)) * W;
        const uint8_t* so = a.old_sh[pc[p].shard] + off;
        const uint8_t* sn = a.new_sh[pc[p].shard] + off;
        if (((reinterpret_cast<uintptr_t>(so) | reinterpret_cast<uintptr_t>(sn)) & 15u) == 0) {
            vo = *reinterpret_cast<const v4u*>(so);
            vn = *reinterpret_cast<const v4u*>(sn);
            return;
        }
    }
    // element by element (group crosses a piece border, is misaligned, or is
    // the tail): shift each element into a 128-bit accumulator
    uint64_t olo = 0, ohi = 0, nlo = 0, nhi = 0;
    for (uint32_t i = 0; i < V; i++) {
        const uint32_t e = e0 + i;
        uint64_t xo = 0, xn = 0;
        if (e < n_c) {
            while (e >= pend) {
                p++;
                pstart = pc[p].canon_start;
                pend = pstart + uint32_t(pc[p].len_m1) + 1;
            }
            const uint64_t off = (pc[p].shard_elem_off + (e - pstart)) * W;
            const uint8_t* so = a.old_sh[pc[p].shard] + off;
            const uint8_t* sn = a.new_sh[pc[p].shard] + off;
            if constexpr (W == 1) { xo = *so; xn = *sn; }
            else if constexpr (W == 2) { xo = *reinterpret_cast<const uint16_t*>(so); xn = *reinterpret_cast<const uint16_t*>(sn); }
            else { xo = *reinterpret_cast<const uint32_t*>(so); xn = *reinterpret_cast<const uint32_t*>(sn); }
        }
        olo = (olo >> (8 * W)) | (ohi << (64 - 8 * W));
        ohi = (ohi >> (8 * W)) | (xo << (64 - 8 * W));
        nlo = (nlo >> (8 * W)) | (nhi << (64 - 8 * W));
        nhi = (nhi >> (8 * W)) | (xn << (64 - 8 * W));
    }
    vo = v4u{uint32_t(olo), uint32_t(olo >> 32), uint32_t(ohi), uint32_t(ohi >> 32)};
    vn = v4u{uint32_t(nlo), uint32_t(nlo >> 32), uint32_t(nhi), uint32_t(nhi >> 32)};
}

// What a workgroup needs to know of its tile (uniform: scalar registers).
struct TileCtx {
    uint64_t c0;             // first canonical element of the chunk
    uint64_t fast_old;       // fast tiles: address of the chunk's old / new bytes
    uint64_t fast_new;
    uint64_t scale_bit_off;
    uint64_t numel;
    uint32_t tile, tensor, chunk_idx, first_piece, n_pieces, n_c, w, route, scale_block, fast, direct;
};

// A fast tile is one aligned piece covering a full chunk: 128-bit loads
// straight from the shard.
__device__ __forceinline__ TileCtx tile_ctx(const EncodeArgs& a, uint32_t tile) {
    TileCtx c;
    const DevChunk ch = uniform_load(a.chunks + tile);
    const DevTensor td = uniform_load(a.tensors + ch.tensor);
    const uint64_t E = kChunkBytes / td.w;
    c.tile = tile;
    c.tensor = ch.tensor;
    c.chunk_idx = ch.chunk_idx;
    c.first_piece = ch.first_piece;
    c.n_pieces = ch.n_pieces & kPiecesMask;
    c.direct = (ch.n_pieces & kChunkDirect) ? 1u : 0u;
    c.c0 = uint64_t(ch.chunk_idx) * E;
    c.n_c = uint32_t(umin64(E, td.numel - c.c0));
    c.w = td.w;
    c.route = td.route;
    c.scale_block = td.scale_block;
    c.scale_bit_off = td.scale_bit_off;
    c.numel = td.numel;
    c.fast = 0;
    c.fast_old = c.fast_new = 0;
    if (c.n_pieces == 1 && c.n_c == E) {
        const DevPiece p0 = uniform_load(a.pieces + ch.first_piece);
        const uint64_t so = uniform_load(reinterpret_cast<const uint64_t*>(a.old_sh) + p0.shard);
        const uint64_t sn = uniform_load(reinterpret_cast<const uint64_t*>(a.new_sh) + p0.shard);
        c.fast_old = so + p0.shard_elem_off * td.w;
        c.fast_new = sn + p0.shard_elem_off * td.w;
        c.fast = ((c.fast_old | c.fast_new) & 15u) == 0 ? 1u : 0u;
    }
    return c;
}

// Issue the 128-bit loads of a fast tile (the registers fill later).
__device__ __forceinline__ void load_fast(const TileCtx& c, v4u (&lo)[kVecsPerThread], v4u (&ln)[kVecsPerThread]) {
    gv4p vo = reinterpret_cast<gv4p>(c.fast_old) + threadIdx.x;
    gv4p vn = reinterpret_cast<gv4p>(c.fast_new) + threadIdx.x;
#pragma unroll
    for (uint32_t k = 0; k < kVecsPerThread; k++) {
        lo[k] = __builtin_nontemporal_load(vo + k * kThreads);
        ln[k] = __builtin_nontemporal_load(vn + k * kThreads);
    }
}

// Gather a tile that spans several pieces (the direct projection).  With few
// pieces, each piece's old / new addresses are resolved once into LDS; every
// group then finds its piece there, all aligned in-piece groups are loaded at
// once, and only groups that straddle pieces are gathered element by element.
template <int W>
__device__ __forceinline__ void gather_tile(const EncodeArgs& a, EncodeShared& S, const TileCtx& c,
                                            v4u (&lo)[kVecsPerThread], v4u (&ln)[kVecsPerThread]) {
    constexpr uint32_t V = 16 / W;
    const uint32_t tid = threadIdx.x;
    const DevPiece* gp = a.pieces + c.first_piece;
    if (c.n_pieces > kMaxCachedPieces) {
#pragma unroll
        for (uint32_t k = 0; k < kVecsPerThread; k++)
            gather_group<W>(a, gp, c.n_pieces, (tid + k * kThreads) * V, c.n_c, lo[k], ln[k]);
        return;
    }
    if (tid < c.n_pieces) {
        const DevPiece p = gp[tid];
        S.pieces[tid] = p;
        S.pstart[tid] = p.canon_start;
        S.pend[tid] = uint32_t(p.canon_start) + uint32_t(p.len_m1) + 1;
        S.pold[tid] = reinterpret_cast<uint64_t>(a.old_sh[p.shard] + p.shard_elem_off * W);
        S.pnew[tid] = reinterpret_cast<uint64_t>(a.new_sh[p.shard] + p.shard_elem_off * W);
    }
    __syncthreads();
    const uint32_t np = c.n_pieces;
    uint32_t direct = 0;
#pragma unroll
    for (uint32_t k = 0; k < kVecsPerThread; k++) {
        const uint32_t e0 = (tid + k * kThreads) * V;
        lo[k] = v4u{0, 0, 0, 0};
        ln[k] = v4u{0, 0, 0, 0};
        if (e0 < c.n_c) {
            uint32_t l = 0, h = np;
            while (h - l > 1) {
                const uint32_t mid = (l + h) >> 1;
                if (S.pstart[mid] <= e0) l = mid;
                else h = mid;
            }
            const uint64_t ao = S.pold[l] + uint64_t(e0 - S.pstart[l]) * W;
            const uint64_t an = S.pnew[l] + uint64_t(e0 - S.pstart[l]) * W;
            if (e0 + V <= S.pend[l] && ((ao | an) & 15u) == 0) {
                lo[k] = __builtin_nontemporal_load(reinterpret_cast<gv4p>(ao));
                ln[k] = __builtin_nontemporal_load(reinterpret_cast<gv4p>(an));
                direct |= 1u << k;
            }
        }
    }
#pragma unroll
    for (uint32_t k = 0; k < kVecsPerThread; k++)
        if (!((direct >> k) & 1u)) gather_group<W>(a, S.pieces, np, (tid + k * kThreads) * V, c.n_c, lo[k], ln[k]);
}

// Per-k routing bits of this thread's groups (1 = overwrite record).  A
// block-scaled group goes to the overwrite record iff the fp32 scale of its
// block changed (a group never straddles blocks: scale_block is a multiple
// of the group's element count).  Called once the tile's own loads are in
// flight; its flag loads are issued together.
template <int W>
__device__ __forceinline__ uint32_t ow_mask(const EncodeArgs& a, const TileCtx& c) {
    constexpr uint32_t V = 16 / W;
    if (a.mode == DCR_MODE_RETRY || c.route == DCR_ROUTE_OVERWRITE) return (1u << kVecsPerThread) - 1;
    if (c.route != DCR_ROUTE_BLOCK_SCALED) return 0;
    const uint32_t tid = threadIdx.x;
    const uint64_t sbg = c.scale_block / V;               // groups per block
    const uint64_t gi = c.c0 / V + tid;                   // this thread's first group in the tensor
    uint64_t q = gi / sbg, r = gi % sbg;
    const uint64_t sq = kThreads / sbg, sr = kThreads % sbg;
    // the flag words of the thread's groups, loaded together (a group past
    // the chunk's elements reads the tensor's first flag word and is masked)
    uint64_t fw[kVecsPerThread];
    uint32_t sh[kVecsPerThread], in = 0;
#pragma unroll
    for (uint32_t k = 0; k < kVecsPerThread; k++) {
        const bool ok = (tid + k * kThreads) * V < c.n_c;
        const uint64_t bit = c.scale_bit_off + (ok ? q : 0);
        fw[k] = a.scale_flags[bit >> 6];
        sh[k] = uint32_t(bit & 63);
        in |= ok ? 1u << k : 0u;
        q += sq;
        r += sr;
        if (r >= sbg) {
            r -= sbg;
            q++;
        }
    }
    uint32_t m = 0;
#pragma unroll
    for (uint32_t k = 0; k < kVecsPerThread; k++) m |= uint32_t((fw[k] >> sh[k]) & 1u) << k;
    return m & in;
}

// 1 in each 16-bit half of the result iff that half of d is nonzero (one
// packed 16-bit integer minimum against 1).
__device__ __forceinline__ uint32_t nz16(uint32_t d) {
    uint32_t r;
    asm("v_pk_min_u16 %0, %1, %2" : "=v"(r) : "v"(d), "s"(0x00010001u));
    return r;
}

// The 8 nonzero flags of the 16-bit halves of d[0..3] as bits 0..7 (half h
// of word i -> bit 2i + h): the flags sit at bits 2i and 2i + 16 after the
// shifts, and folding bit 16 + 2i onto 2i + 1 packs them.
__device__ __forceinline__ uint32_t pack_nz16(uint32_t m0, uint32_t m1, uint32_t m2, uint32_t m3) {
    const uint32_t x = m0 | (m1 << 2) | (m2 << 4) | (m3 << 6);
    return (x | (x >> 15)) & 0xFFu;
}

// Changed-element bits of a 16-byte group of W-byte elements (d = old ^ new,
// four 32-bit words); for W = 2 also the bits of elements whose high byte
// changed.  Integer arithmetic only (for bytes: x != 0 for an n-bit field x
// is (x + 2^n - 1) >> n).
template <int W>
__device__ __forceinline__ uint32_t changed_bits(const uint32_t (&d)[4], uint32_t& hi_bits) {
    if constexpr (W == 2) {
        hi_bits = pack_nz16(nz16(d[0] & 0xFF00FF00u), nz16(d[1] & 0xFF00FF00u), nz16(d[2] & 0xFF00FF00u),
                            nz16(d[3] & 0xFF00FF00u));
        return pack_nz16(nz16(d[0]), nz16(d[1]), nz16(d[2]), nz16(d[3]));
    }
    uint32_t b = 0, h = 0;
#pragma unroll
    for (uint32_t i = 0; i < 4; i++) {
        const uint32_t x = d[i];
        if constexpr (W == 4) {
            b |= uint32_t(x != 0) << i;
        } else {
            // high bit of each byte set iff the byte is nonzero
            const uint32_t t = (((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) & 0x80808080u;
            b |= ((t >> 7) & 1u) << (4 * i);
            b |= ((t >> 15) & 1u) << (4 * i + 1);
            b |= ((t >> 23) & 1u) << (4 * i + 2);
            b |= ((t >> 31) & 1u) << (4 * i + 3);
        }
    }
    hi_bits = h;
    return b;
}

// Compare stored bits and route each 16-byte group: meta[k] = changed bits |
// high-byte bits << 16 | kind << 31; cnt = per-k counts packed 16 bits per k
// (XOR K, overwrite K, XOR high bytes); the group's payload words (XOR mask or
// new bits) go to S.pw.
template <int W>
__device__ __forceinline__ void digest_tile(EncodeShared& S, uint32_t owm, const v4u (&lo)[kVecsPerThread],
                                            const v4u (&ln)[kVecsPerThread], uint32_t (&meta)[kVecsPerThread],
                                            uint64_t (&cnt)[3]) {
    const uint32_t tid = threadIdx.x;
    uint32_t kx = 0, ko = 0, kh = 0;   // per-k counts, 8 bits each
#pragma unroll
    for (uint32_t k = 0; k < kVecsPerThread; k++) {
        const uint32_t g = tid + k * kThreads;
        const uint32_t d[4] = {lo[k].x ^ ln[k].x, lo[k].y ^ ln[k].y, lo[k].z ^ ln[k].z, lo[k].w ^ ln[k].w};
        uint32_t h;
        const uint32_t b = changed_bits<W>(d, h);
        const uint32_t kd = (owm >> k) & 1u;
        if (b) {
            const v4u q = kd == DCR_KIND_XOR ? v4u{d[0], d[1], d[2], d[3]} : ln[k];
            *reinterpret_cast<v4u*>(S.pw[g]) = q;
        }
        if (kd != DCR_KIND_XOR) h = 0;
        meta[k] = b | (h << 16) | (kd << 31);
        const uint32_t pb = uint32_t(__popc(b)) << (8 * k);
        kx |= kd == DCR_KIND_XOR ? pb : 0u;
        ko |= kd == DCR_KIND_XOR ? 0u : pb;
        kh |= uint32_t(__popc(h)) << (8 * k);
    }
    // widened once to the scan's 16-bit fields
    auto widen = [](uint32_t x) {
        return uint64_t(x & 0xFFu) | (uint64_t((x >> 8) & 0xFFu) << 16) | (uint64_t((x >> 16) & 0xFFu) << 32) |
               (uint64_t(x >> 24) << 48);
    };
    cnt[0] = widen(kx);
    cnt[1] = widen(ko);
    cnt[2] = widen(kh);
}

// Tile totals and, per k, the totals of all lower k (uniform).
struct TileSums {
    uint32_t Kx, Ko, Hx;
    uint32_t kb[3][kVecsPerThread];
};

// Workgroup scan of the packed counts: cnt becomes each thread's exclusive
// prefix; its barriers also publish S.pw.
__device__ __forceinline__ TileSums scan_tile(EncodeShared& S, uint64_t (&cnt)[3]) {
    uint64_t tot[3];
    block_excl_scan<3>(cnt, tot, S.scan);
    TileSums t;
    t.Kx = t.Ko = t.Hx = 0;
#pragma unroll
    for (uint32_t k = 0; k < kVecsPerThread; k++) {
        t.kb[0][k] = t.Kx;
        t.kb[1][k] = t.Ko;
        t.kb[2][k] = t.Hx;
        t.Kx += sgpr(field16(tot[0], k));
        t.Ko += sgpr(field16(tot[1], k));
        t.Hx += sgpr(field16(tot[2], k));
    }
    return t;
}

// One output window [w0, w0 + kWinBytes) of a tile's records: each thread
// puts the bitmap bits of its groups and the plane bytes of its changed
// elements that fall in the window into LDS (zeroed first: the zero padding),
// then the window leaves as 128-bit stores.  ONE: the records fit in one
// window (no range checks).
template <int W, bool ONE, class Dest>
__device__ __forceinline__ void write_window(EncodeShared& S, const Dest& dest, uint32_t w0,
                                             uint32_t total, uint32_t bm, const uint32_t (&meta)[kVecsPerThread],
                                             const uint64_t (&cnt)[3], const TileSums& t, const RecLayout& L) {
    constexpr uint32_t V = 16 / W;
    const uint32_t tid = threadIdx.x;
    const uint32_t Kx = t.Kx, Ko = t.Ko;
    const uint32_t base_o = L.size_x;
    const uint32_t pkx = dpad16(Kx), pko = dpad16(Ko);
    // records in bitmap layout, non-empty (uniform)
    const uint32_t bmx = sgpr(L.list_x ? 0u : Kx), bmo = sgpr(L.list_o ? 0u : Ko);
    const uint32_t hi_x_dense = sgpr(L.mode_x == DCR_HI_DENSE ? 1u : 0u);
    const uint32_t hi_x_sparse = sgpr(L.mode_x == DCR_HI_SPARSE ? 1u : 0u);
    const uint32_t w1 = w0 + kWinBytes;
    uint8_t* win = S.win;
    for (uint32_t q = tid; q < kWinBytes / 16; q += kThreads) reinterpret_cast<v4u*>(win)[q] = v4u{0, 0, 0, 0};
    __syncthreads();
    auto inwin = [&](uint32_t pos) { return ONE || (pos >= w0 && pos < w1); };
    auto put = [&](uint32_t pos, uint32_t v) {
        if (inwin(pos)) win[pos - w0] = uint8_t(v);
    };
    // pos is even and windows start at multiples of kWinBytes: both bytes
    // share the window
    auto put16 = [&](uint32_t pos, uint32_t v) {
        if (inwin(pos)) *reinterpret_cast<uint16_t*>(win + (pos - w0)) = uint16_t(v);
    };
#pragma unroll
    for (uint32_t k = 0; k < kVecsPerThread; k++) {
        const uint32_t g = tid + k * kThreads;
        uint32_t b = meta[k] & 0xFFFFu;
        const bool x = (meta[k] >> 31) == DCR_KIND_XOR;
        // change bitmaps (LSB first) of both records, padding included
        const uint32_t bx = x ? b : 0u, bo = x ? 0u : b;
        uint32_t px = 0, po = 0;
        if constexpr (W == 4) {      // nibble pairs: the odd lane's bits go to the even lane
            px = __shfl_xor(bx, 1, 64);
            po = __shfl_xor(bo, 1, 64);
        }
        if (g * V < bm * 8) {
            if constexpr (W == 2) {
                if (bmx) put(g, bx);
                if (bmo) put(base_o + g, bo);
            } else if constexpr (W == 1) {
                if (bmx) { put(2 * g, bx); put(2 * g + 1, bx >> 8); }
                if (bmo) { put(base_o + 2 * g, bo); put(base_o + 2 * g + 1, bo >> 8); }
            } else {
                if ((g & 1) == 0) {
                    if (bmx) put(g / 2, bx | (px << 4));
                    if (bmo) put(base_o + g / 2, bo | (po << 4));
                }
            }
        }
        if (!b) continue;
        const uint32_t rb = x ? 0u : base_o;
        const uint32_t pk = x ? pkx : pko;
        const uint32_t lst = ONE ? (x ? L.list_x : L.list_o) : 0u;   // several windows: lists written after

        const uint32_t lo = rb + (x ? L.head_x : L.head_o);
        uint32_t j = x ? t.kb[0][k] + field16(cnt[0], k) : t.kb[1][k] + field16(cnt[1], k);
        uint32_t hr = t.kb[2][k] + field16(cnt[2], k);
        if (!ONE) {
            // every byte of this group lies in [start, end): skip the group
            // when that range misses the window
            const uint32_t nb = uint32_t(__popc(b));
            uint32_t end = lo + (W - 1) * pk + j + nb;
            if (W == 2 && x)
                end = hi_x_sparse ? L.off_hi_x + hr + nb : (hi_x_dense ? L.off_hi_x + j + nb : lo + j + nb);
            if (lo + j >= w1 || end <= w0) continue;
        }
        const v4u q = *reinterpret_cast<const v4u*>(S.pw[g]);
        // byte planes of the group packed into 64-bit values
        uint64_t pl0 = 0, ph = 0;
        if constexpr (W == 2) {
            const uint32_t qq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (uint32_t i = 0; i < 8; i++) {
                const uint32_t e = (qq[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
                pl0 |= uint64_t(e & 0xFFu) << (8 * i);
                ph |= uint64_t(e >> 8) << (8 * i);
            }
        } else {
            const uint32_t qq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (uint32_t i = 0; i < 4; i++) {
                pl0 |= uint64_t(qq[i] & 0xFFu) << (8 * i);
                pl0 |= uint64_t((qq[i] >> 8) & 0xFFu) << (32 + 8 * i);
                ph |= uint64_t((qq[i] >> 16) & 0xFFu) << (8 * i);
                ph |= uint64_t(qq[i] >> 24) << (32 + 8 * i);
            }
        }
#pragma nounroll
        while (b) {
            const uint32_t i = uint32_t(__ffs(b) - 1);
            b &= b - 1;
            if (lst) put16(rb + 2 * j, g * V + i);
            if constexpr (W == 1) {
                // byte i of the group: 32-bit selects and shifts only
                const uint32_t wv = (i & 8u) ? ((i & 4u) ? q.w : q.z) : ((i & 4u) ? q.y : q.x);
                put(lo + j, wv >> (8u * (i & 3u)));
            } else if constexpr (W == 2) {
                put(lo + j, uint32_t(pl0 >> (8 * i)));
                const uint32_t hb = uint32_t(ph >> (8 * i)) & 0xFFu;
                if (!x) {
                    put(lo + pk + j, hb);
                } else if (hi_x_dense) {
                    put(L.off_hi_x + j, hb);
                } else if (hi_x_sparse && hb) {
                    // presence bit j (LSB first) and the byte itself
                    const uint32_t pp = L.off_pres + (j >> 3);
                    if (inwin(pp)) atomicOr(reinterpret_cast<uint32_t*>(win) + ((pp - w0) >> 2), 1u << (j & 31));
                    put(L.off_hi_x + hr, hb);
                    hr++;
                }
            } else {
                put(lo + j, uint32_t(pl0 >> (8 * i)));
                put(lo + pk + j, uint32_t(pl0 >> (32 + 8 * i)));
                put(lo + 2 * pk + j, uint32_t(ph >> (8 * i)));
                put(lo + 3 * pk + j, uint32_t(ph >> (32 + 8 * i)));
            }
            j++;
        }
    }
    __syncthreads();
    // where the window goes, decided now by every thread (uniform); nowhere:
    // nothing is copied out
    uint8_t* const out = dest.at(S, w0);
    if constexpr (Dest::kMaySkip) {
        if (!out) return;
    }
    // non-temporal 128-bit stores: the records are read back only after the
    // whole grid (by the fix-up, or by the stream's consumer).  Index lists
    // of records spanning several windows are stored over these bytes after
    // the last window: plain stores then, ordered by the barrier in between.
    const uint32_t n = ONE ? total : uint32_t(umin64(kWinBytes, total - w0));
    if (ONE || !(L.list_x | L.list_o)) {
        for (uint32_t q = opaque_tid(); q < n / 16; q += kThreads)
            __builtin_nontemporal_store(reinterpret_cast<const v4u*>(win)[q], reinterpret_cast<v4u*>(out + w0) + q);
    } else {
        for (uint32_t q = opaque_tid(); q < n / 16; q += kThreads)
            reinterpret_cast<v4u*>(out + w0)[q] = reinterpret_cast<const v4u*>(win)[q];
    }
}

// Where a tile's records go.  The record writer calls begin() (every
// thread) before the first window and at(S, w0) (every thread, uniform
// result) once a window's bytes are in LDS; with kMaySkip, nullptr means
// nowhere: nothing is copied out.
struct SlotDest {   // a fixed address: the tile's staging slot or its place in the payload
    static constexpr bool kMaySkip = false;
    uint8_t* out;
    __device__ __forceinline__ void begin(EncodeShared&) const {}
    __device__ __forceinline__ uint8_t* at(EncodeShared&, uint32_t) const { return out; }
};

// Compact staging: the records go to the offset thread 0 claims first in its
// workgroup's partition of the staging area (one atomic add on one of
// kStageParts counters, so no single address takes every tile's atomic); the
// claim is recorded for the fix-up, and a claim past the partition's end
// (kNoClaim) writes nothing: the fix-up lists the tile to be encoded again at
// its place.  The atomic's latency overlaps the window's zeroing; the offset
// is read from LDS (published by the window's barrier) when it is copied out.
struct CompactDest {
    static constexpr bool kMaySkip = true;
    const EncodeArgs& a;
    uint32_t tile, total;
    __device__ __forceinline__ void begin(EncodeShared& S) const {
        if (threadIdx.x == 0) {
            const uint32_t part = blockIdx.x & (kStageParts - 1);
            const uint64_t o = atomicAdd(a.stage_ctr + part, (unsigned long long)total);
            const uint64_t cl = o + total <= a.part_bytes ? uint64_t(part) * a.part_bytes + o : kNoClaim;
            a.soff[tile] = cl;
            S.claim = cl;
        }
    }
    __device__ __forceinline__ uint8_t* at(EncodeShared& S, uint32_t) const {
        const uint64_t cl = S.claim;
        return cl == kNoClaim ? nullptr : a.stage + cl;
    }
};

// In order: the tile's place in the payload, from the decoupled look-back,
// run by wave 0 once the first window is in LDS (the wait for predecessors
// that have not yet published overlaps the window's assembly); S.excl holds
// the tile's exclusive prefix, and nullptr means the records do not fit the
// caller's buffers (nothing written).
struct LookBackDest {
    static constexpr bool kMaySkip = true;
    const EncodeArgs& a;
    uint32_t tile;
    uint64_t agg;
    __device__ __forceinline__ void begin(EncodeShared&) const {}
    __device__ __forceinline__ uint8_t* at(EncodeShared& S, uint32_t w0) const {
        if (w0 == 0) {
            if (threadIdx.x < 64) {
                const uint64_t excl = look_back(a.status, tile, threadIdx.x);
                if (threadIdx.x == 0) {
                    if (tile > 0) st_status(a.status + tile, ((excl + agg) << kValShift) | kFlagIncl);
                    S.excl = excl;
                    const uint64_t R = excl >> kRecShift, P = (excl & kP16Mask) << 4;
                    const bool fits = (R + (agg >> kRecShift)) * DCR_DIRENT_BYTES <= a.dir_cap &&
                                      P + ((agg & kP16Mask) << 4) <= a.payload_cap;
                    S.claim = fits ? reinterpret_cast<uint64_t>(a.payload) + P : 0;
                }
            }
            __syncthreads();
        }
        return reinterpret_cast<uint8_t*>(S.claim);
    }
};

// Write a tile's records (XOR record, then overwrite record) where dest
// says: change bitmaps (LSB first), byte planes of the changed elements in
// element order, zero padding to 16 bytes, assembled in LDS one window at a
// time.
template <int W, class Dest>
__device__ __forceinline__ void write_tile(EncodeShared& S, const Dest& dest, uint32_t n_c,
                                           const uint32_t (&meta)[kVecsPerThread], const uint64_t (&cnt)[3],
                                           const TileSums& t, const RecLayout& L) {
    const uint32_t bm = dpad16((n_c + 7) / 8);
    const uint32_t total = L.size_x + L.size_o;
    dest.begin(S);
    if (total <= kWinBytes) {
        write_window<W, true>(S, dest, 0, total, bm, meta, cnt, t, L);
        return;
    }
#pragma nounroll
    for (uint32_t w0 = 0; w0 < total; w0 += kWinBytes) {
        // keep the per-group values inside the loop (recomputed per window)
        uint32_t m[kVecsPerThread];
        uint64_t cc[3];
#pragma unroll
        for (uint32_t k = 0; k < kVecsPerThread; k++) m[k] = __builtin_amdgcn_readfirstlane(0) + meta[k];
        cc[0] = cnt[0];
        cc[1] = cnt[1];
        cc[2] = cnt[2];
        asm volatile("" : "+v"(m[0]), "+v"(m[1]), "+v"(m[2]), "+v"(m[3]), "+v"(cc[0]), "+v"(cc[1]), "+v"(cc[2]));
        write_window<W, false>(S, dest, w0, total, bm, m, cc, t, L);
        __syncthreads();
    }
    uint8_t* const out = dest.at(S, total);
    if constexpr (Dest::kMaySkip) {
        if (!out) return;   // uniform
    }
    // index lists of records spanning several windows: the windows left their
    // bytes zero; each thread stores its changes' indices over them (the
    // barrier above orders these stores after the window copies)
    if (L.list_x || L.list_o) {
        constexpr uint32_t V = 16 / W;
#pragma unroll
        for (uint32_t k = 0; k < kVecsPerThread; k++) {
            uint32_t b = meta[k] & 0xFFFFu;
            const bool x = (meta[k] >> 31) == DCR_KIND_XOR;
            if (!b || !(x ? L.list_x : L.list_o)) continue;
            const uint32_t g = threadIdx.x + k * kThreads;
            uint16_t* dst = reinterpret_cast<uint16_t*>(out + (x ? 0u : L.size_x));
            uint32_t j = x ? t.kb[0][k] + field16(cnt[0], k) : t.kb[1][k] + field16(cnt[1], k);
            while (b) {
                const uint32_t i = uint32_t(__ffs(b) - 1);
                b &= b - 1;
                dst[j++] = uint16_t(g * V + i);
            }
        }
    }
}

__device__ __forceinline__ uint64_t tile_aggregate(const TileSums& t, const RecLayout& L) {
    const uint32_t nrec = (t.Kx ? 1u : 0u) + (t.Ko ? 1u : 0u);
    return (uint64_t(nrec) << kRecShift) | ((L.size_x + L.size_o) >> 4);
}
__device__ __forceinline__ uint64_t tile_counts(const TileSums& t) {
    return uint64_t(t.Kx) | (uint64_t(t.Ko) << 17) | (uint64_t(t.Hx) << 34);
}

// Partial retry: whether the tile is to be encoded (every tile without a
// wanted-chunk mask).  Uniform.
__device__ __forceinline__ bool tile_wanted(const EncodeArgs& a, uint32_t tile) {
    return !a.need || ((uniform_load(a.need + (tile >> 6)) >> (tile & 63u)) & 1u) != 0;
}

// A tile left out of a partial retry: no records, no changes (and, in order,
// an empty aggregate for the look-back).
__device__ __forceinline__ void skip_tile(const EncodeArgs& a, uint32_t tile, bool publish) {
    if (threadIdx.x == 0) {
        if (publish) st_status(a.status + tile, tile == 0 ? kFlagIncl : kFlagAgg);
        a.tile_agg[tile] = 0;
        a.tile_info[tile] = 0;
    }
}

// In-order encode of one tile of W-byte elements (no staging area): publish
// the aggregate, write the records in place (the look-back for the tile's
// exclusive prefix runs once the first window is assembled), then the
// directory entries.
template <int W>
__device__ __forceinline__ void inorder_tile(const EncodeArgs& a, EncodeShared& S, const TileCtx& c) {
    const uint32_t tid = threadIdx.x;
    v4u lo[kVecsPerThread], ln[kVecsPerThread];
    if (c.fast) load_fast(c, lo, ln);
    else gather_tile<W>(a, S, c, lo, ln);
    const uint32_t owm = ow_mask<W>(a, c);   // after the tile's loads are issued
    uint32_t meta[kVecsPerThread];
    uint64_t cnt[3];
    digest_tile<W>(S, owm, lo, ln, meta, cnt);
    const TileSums t = scan_tile(S, cnt);
    const RecLayout L = rec_layout(W, c.n_c, t.Kx, t.Ko, t.Hx, a.lists);
    const uint64_t agg = tile_aggregate(t, L);
    const uint32_t nrec = uint32_t(agg >> kRecShift);
    const uint32_t tile = c.tile;
    if (tid == 0) {
        st_status(a.status + tile, (agg << kValShift) | (tile == 0 ? kFlagIncl : kFlagAgg));
        a.tile_agg[tile] = agg;
        a.tile_info[tile] = tile_counts(t);
    }
    if (nrec == 0) return;   // uniform; an empty tile's aggregate is all it owes
    // the look-back runs once the first window is assembled
    write_tile<W>(S, LookBackDest{a, tile, agg}, c.n_c, meta, cnt, t, L);
    if (!S.claim) return;   // uniform: the records do not fit the caller's buffers
    const uint64_t R = S.excl >> kRecShift;
    const uint64_t P = (S.excl & kP16Mask) << 4;
    if (tid < nrec) put_dirent(a.dir, R + tid, tid, c.tensor, c.chunk_idx, W, L, t.Kx, t.Ko, P);
}

// In-order encode (no staging area): one workgroup per tile, tiles claimed
// in increasing order from a counter, so every tile a look-back waits on
// belongs to a workgroup that is already running.  WIDTHS: the element
// widths of the plan's tiles (1 | 2 | 4): only their code is built (the
// three together spill heavily).
template <int WIDTHS>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(8, 8))) void encode_kernel(EncodeArgs a) {
    __shared__ EncodeShared S;
    if (threadIdx.x == 0) S.next = atomicAdd(a.counter + kCtrTile, 1u);
    __syncthreads();
    const uint32_t tile = sgpr(S.next);
    if (tile >= a.n_tiles) return;
    if (!tile_wanted(a, tile)) {
        skip_tile(a, tile, true);
        return;
    }
    const TileCtx c = tile_ctx(a, tile);
    if constexpr (WIDTHS == 1 || WIDTHS == 2 || WIDTHS == 4) {
        inorder_tile<WIDTHS>(a, S, c);
    } else {
        if ((WIDTHS & 2) && c.w == 2) inorder_tile<2>(a, S, c);
        else if ((WIDTHS & 1) && c.w == 1) inorder_tile<1>(a, S, c);
        else if (WIDTHS & 4) inorder_tile<4>(a, S, c);
    }
}

// Staged encode of one tile of W-byte elements: write the records to the
// tile's slot of the staging area; nothing waits on another workgroup.
template <int W>
__device__ __forceinline__ void staged_tile(const EncodeArgs& a, EncodeShared& S, const TileCtx& c) {
    const uint32_t tid = threadIdx.x;
    v4u lo[kVecsPerThread], ln[kVecsPerThread];
    if (c.fast) load_fast(c, lo, ln);
    else gather_tile<W>(a, S, c, lo, ln);
    const uint32_t owm = ow_mask<W>(a, c);   // after the tile's loads are issued
    uint32_t meta[kVecsPerThread];
    uint64_t cnt[3];
    digest_tile<W>(S, owm, lo, ln, meta, cnt);
    const TileSums t = scan_tile(S, cnt);
    const RecLayout L = rec_layout(W, c.n_c, t.Kx, t.Ko, t.Hx, a.lists);
    const uint64_t agg = tile_aggregate(t, L);
    if (tid == 0) {
        a.tile_agg[c.tile] = agg;
        a.tile_info[c.tile] = tile_counts(t);
    }
    if (!agg) return;
    if (a.compact) write_tile<W>(S, CompactDest{a, c.tile, L.size_x + L.size_o}, c.n_c, meta, cnt, t, L);
    else write_tile<W>(S, SlotDest{a.stage + a.slots[c.tile]}, c.n_c, meta, cnt, t, L);
}

// A tile encoded again, straight to its place in the payload (compact
// staging found no room for it in the first pass): the same records, no
// aggregates published.
template <int W>
__device__ __forceinline__ void redo_tile(const EncodeArgs& a, EncodeShared& S, const TileCtx& c, uint8_t* out) {
    v4u lo[kVecsPerThread], ln[kVecsPerThread];
    if (c.fast) load_fast(c, lo, ln);
    else gather_tile<W>(a, S, c, lo, ln);
    const uint32_t owm = ow_mask<W>(a, c);   // after the tile's loads are issued
    uint32_t meta[kVecsPerThread];
    uint64_t cnt[3];
    digest_tile<W>(S, owm, lo, ln, meta, cnt);
    const TileSums t = scan_tile(S, cnt);
    const RecLayout L = rec_layout(W, c.n_c, t.Kx, t.Ko, t.Hx, a.lists);
    if (t.Kx || t.Ko) write_tile<W>(S, SlotDest{out}, c.n_c, meta, cnt, t, L);
}

// Staged encode of the tiles that are not direct (pieces that split
// 16-byte groups, misaligned or many pieces, ragged tails): one workgroup
// per listed tile.
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(8, 8))) void encode_slow_kernel(
    EncodeArgs a, const uint32_t* tiles, uint32_t n) {
    __shared__ EncodeShared S;
    if (blockIdx.x >= n) return;
    const uint32_t tile = tiles[blockIdx.x];
    if (!tile_wanted(a, tile)) return;   // the fix-up counts it as empty
    const TileCtx c = tile_ctx(a, tile);
    if (c.w == 2) staged_tile<2>(a, S, c);
    else if (c.w == 1) staged_tile<1>(a, S, c);
    else staged_tile<4>(a, S, c);
}

// Issue the loads of a direct tile: straight 128-bit loads for a fast tile;
// otherwise each group finds its piece in an LDS copy of the piece table
// (every group is inside one piece and aligned).  Ends with a barrier when it
// used the LDS table.
__device__ __forceinline__ void prefetch_direct(const EncodeArgs& a, EncodeShared& S, const TileCtx& c,
                                                v4u (&o)[kVecsPerThread], v4u (&n)[kVecsPerThread]) {
    if (c.fast) {
        load_fast(c, o, n);
        return;
    }
    const uint32_t tid = threadIdx.x;
    const uint32_t w = c.w, V = 16u / w, np = c.n_pieces;
    if (tid < np) {
        const DevPiece p = a.pieces[c.first_piece + tid];
        S.pstart[tid] = p.canon_start;
        S.pold[tid] = reinterpret_cast<uint64_t>(a.old_sh[p.shard]) + p.shard_elem_off * w;
        S.pnew[tid] = reinterpret_cast<uint64_t>(a.new_sh[p.shard]) + p.shard_elem_off * w;
    }
    __syncthreads();
#pragma unroll
    for (uint32_t k = 0; k < kVecsPerThread; k++) {
        const uint32_t e0 = (tid + k * kThreads) * V;
        o[k] = v4u{0, 0, 0, 0};
        n[k] = v4u{0, 0, 0, 0};
        if (e0 < c.n_c) {
            uint32_t l = 0, h = np;
            while (h - l > 1) {
                const uint32_t mid = (l + h) >> 1;
                if (S.pstart[mid] <= e0) l = mid;
                else h = mid;
            }
            const uint64_t off = uint64_t(e0 - S.pstart[l]) * w;
            o[k] = __builtin_nontemporal_load(reinterpret_cast<gv4p>(S.pold[l] + off));
            n[k] = __builtin_nontemporal_load(reinterpret_cast<gv4p>(S.pnew[l] + off));
        }
    }
    __syncthreads();   // the LDS piece table is free again
}

// Staged encode of the direct tiles of W-byte elements (the staging area
// holds every chunk's slot): one workgroup per list entry; nothing waits on
// another workgroup.
template <int W, bool LISTS, bool COMPACT>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(8, 8))) void encode_direct_kernel(
    EncodeArgs a, const uint32_t* list, uint32_t n_list) {
    __shared__ EncodeShared S;
    if (blockIdx.x >= n_list) return;
    const uint32_t tid = threadIdx.x;
    if (!tile_wanted(a, list[blockIdx.x])) return;   // the fix-up counts it as empty
    const TileCtx c = tile_ctx(a, list[blockIdx.x]);
    // the slot's address is uniform: read it before this workgroup stores
    // anything, into scalar registers
    uint8_t* const out = a.stage + uniform_load(a.slots + c.tile);
    v4u o[kVecsPerThread], n[kVecsPerThread];
    prefetch_direct(a, S, c, o, n);
    // the tile's loads are in flight: its routing flags next (loaded before,
    // their waits held the tile's loads back)
    const uint32_t owm = ow_mask<W>(a, c);
    uint32_t meta[kVecsPerThread];
    uint64_t cnt[3];
    digest_tile<W>(S, owm, o, n, meta, cnt);
    const TileSums t = scan_tile(S, cnt);
    // LISTS is a.lists as a constant: without index lists every list path
    // folds away
    const RecLayout L = rec_layout(W, c.n_c, t.Kx, t.Ko, t.Hx, LISTS ? 1u : 0u);
    const uint64_t agg = tile_aggregate(t, L);
    if (tid == 0) {
        a.tile_agg[c.tile] = agg;
        a.tile_info[c.tile] = tile_counts(t);
    }
    if (!agg) return;   // uniform
    if constexpr (COMPACT) write_tile<W>(S, CompactDest{a, c.tile, L.size_x + L.size_o}, c.n_c, meta, cnt, t, L);
    else write_tile<W>(S, SlotDest{out}, c.n_c, meta, cnt, t, L);
}

// Compact staging, after the fix-up: the tiles whose records found no room
// in the staging area, encoded again straight to the payload offset the
// fix-up stored for them.  A persistent grid over the fix-up's list (its
// length read once; every workgroup leaves when the list is done), one
// launch per element width, each encoding the listed tiles of its width
// (so each width's code is compiled on its own, free of register spills).
template <int W>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(8, 8))) void encode_redo_kernel(
    EncodeArgs a, const uint32_t* redo, const uint32_t* redo_count) {
    __shared__ EncodeShared S;
    const uint32_t n = sgpr(*redo_count);
    for (uint32_t i = blockIdx.x; i < n; i += gridDim.x) {
        const uint32_t tile = sgpr(redo[i]);
        const TileCtx c = tile_ctx(a, tile);
        if (c.w != W) continue;   // uniform
        uint8_t* out = a.payload + uniform_load(a.soff + tile);
        redo_tile<W>(a, S, c, out);
        __syncthreads();
    }
}

// Encode fix-up: one workgroup of 256 threads per kFixTiles consecutive
// tiles.  Scans the tiles' aggregates (records, payload/16) into exclusive
// prefixes (a short decoupled look-back across fix-up blocks), sums the
// changed elements, and in a staged launch moves every tile's records from
// its slot to their place in the payload and writes their directory
// entries.  The last block stores the stream totals.
struct FixArgs {
    const DevTensor* tensors;
    const DevChunk* chunks;
    const uint64_t* tile_agg;
    const uint64_t* tile_info;
    const uint64_t* slots;
    const uint64_t* need;      // partial retry: wanted-chunk bits (others count as empty), else NULL
    uint64_t* soff;            // compact staging: per-tile staging offsets (kNoClaim: encode again)
    uint32_t* redo;            // compact staging: the tiles to encode again
    uint32_t* redo_count;
    uint64_t* fix_status;
    uint32_t* counter;
    const uint8_t* stage;
    uint8_t* dir;
    uint8_t* payload;
    uint64_t dir_cap;
    uint64_t payload_cap;
    uint32_t n_tiles;
    uint32_t n_blocks;
    uint32_t staged;
    uint32_t lists;
    uint32_t compact;
};

__global__ __launch_bounds__(256) void encode_fixup_kernel(FixArgs a) {
    constexpr uint32_t NW = kFixTiles / 64;
    __shared__ uint64_t wtot[NW], wchg[NW];
    __shared__ uint64_t excl_of[kFixTiles];
    __shared__ uint32_t list[kFixTiles];
    __shared__ uint32_t wcnt[NW];
    __shared__ uint64_t bexcl;
    __shared__ uint32_t blk_s;
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    if (tid == 0) blk_s = atomicAdd(a.counter + kCtrFix, 1u);
    __syncthreads();
    const uint32_t blk = sgpr(blk_s);
    const uint32_t t = blk * kFixTiles + tid;
    const bool in = t < a.n_tiles && (!a.need || ((a.need[t >> 6] >> (t & 63u)) & 1u));
    const uint64_t v = in ? a.tile_agg[t] : 0;
    const uint64_t info = in ? a.tile_info[t] : 0;
    const uint64_t inc = wave_incl_scan(v, lane);
    const uint64_t chg = wave_sum((info & 0x1FFFFu) + ((info >> 17) & 0x1FFFFu));
    const bool staged = a.staged && v != 0;
    const uint64_t sm = __ballot(staged);
    if (lane == 63) wtot[wave] = inc;
    if (lane == 0) {
        wcnt[wave] = uint32_t(__popcll(sm));
        wchg[wave] = chg;
    }
    __syncthreads();
    uint64_t wpre = 0, total = 0;
    uint32_t lpre = 0, nlist = 0;
#pragma unroll
    for (uint32_t w = 0; w < NW; w++) {
        wpre += w < wave ? wtot[w] : 0;
        total += wtot[w];
        lpre += w < wave ? wcnt[w] : 0;
        nlist += wcnt[w];
    }
    if (tid < 64) {
        if (tid == 0) st_status(a.fix_status + blk, (total << kValShift) | (blk == 0 ? kFlagIncl : kFlagAgg));
        const uint64_t ex = look_back(a.fix_status, blk, tid);
        if (tid == 0) {
            if (blk > 0) st_status(a.fix_status + blk, ((ex + total) << kValShift) | kFlagIncl);
            bexcl = ex;
            uint64_t c = 0;
            for (uint32_t w = 0; w < NW; w++) c += wchg[w];
            if (c) atomicAdd(reinterpret_cast<unsigned long long*>(a.counter + kCtrChanged), (unsigned long long)c);
            if (blk == a.n_blocks - 1) *reinterpret_cast<uint64_t*>(a.counter + kCtrTotal) = ex + total;
        }
    }
    __syncthreads();
    excl_of[tid] = bexcl + wpre + inc - v;
    if (staged) list[lpre + uint32_t(__popcll(sm & ((uint64_t(1) << lane) - 1)))] = tid;
    __syncthreads();
    // one wave per staged tile
    for (uint32_t i = wave; i < nlist; i += NW) {
        const uint32_t lt = sgpr(list[i]);
        const uint32_t tile = blk * kFixTiles + lt;
        const uint64_t ex = excl_of[lt];
        const uint64_t R = ex >> kRecShift, P = (ex & kP16Mask) << 4;
        const uint64_t ag = a.tile_agg[tile];
        const uint32_t nrec = uint32_t(ag >> kRecShift);
        const uint64_t bytes = (ag & kP16Mask) << 4;
        if ((R + nrec) * DCR_DIRENT_BYTES > a.dir_cap || P + bytes > a.payload_cap) continue;
        const uint64_t so = a.compact ? a.soff[tile] : a.slots[tile];
        if (so == kNoClaim) {
            // no room in the staging area: encoded again at P after this pass
            if (lane == 0) {
                a.redo[atomicAdd(a.redo_count, 1u)] = tile;
                a.soff[tile] = P;
            }
        } else {
            const v4u* src = reinterpret_cast<const v4u*>(a.stage + so);
            v4u* dst = reinterpret_cast<v4u*>(a.payload + P);
            const uint32_t nv = uint32_t(bytes >> 4);
            uint32_t j = lane;
            for (; j + 192 < nv; j += 256) {
                const v4u q0 = src[j], q1 = src[j + 64], q2 = src[j + 128], q3 = src[j + 192];
                dst[j] = q0;
                dst[j + 64] = q1;
                dst[j + 128] = q2;
                dst[j + 192] = q3;
            }
            for (; j < nv; j += 64) dst[j] = src[j];
        }
        if (lane < nrec) {
            const DevChunk ch = a.chunks[tile];
            const DevTensor td = a.tensors[ch.tensor];
            const uint64_t tinfo = a.tile_info[tile];
            const uint32_t Kx = uint32_t(tinfo & 0x1FFFFu), Ko = uint32_t((tinfo >> 17) & 0x1FFFFu);
            const uint32_t Hx = uint32_t((tinfo >> 34) & 0x1FFFFu);
            const uint64_t E = kChunkBytes / td.w;
            const uint32_t n_c = uint32_t(umin64(E, td.numel - uint64_t(ch.chunk_idx) * E));
            const RecLayout L = rec_layout(td.w, n_c, Kx, Ko, Hx, a.lists);
            put_dirent(a.dir, R + lane, lane, ch.tensor, ch.chunk_idx, td.w, L, Kx, Ko, P);
        }
    }
}

// Per-element "scale bits changed" flags of the scale tensors that gate
// block-scaled tensors.  One workgroup of 256 per scale chunk.
__global__ __launch_bounds__(256) void scale_flags_kernel(const DevTensor* tensors, const DevChunk* chunks,
                                                          const DevPiece* pieces, const uint32_t* scale_chunks,
                                                          const uint8_t* const* old_sh, const uint8_t* const* new_sh,
                                                          uint64_t* flags) {
    const DevChunk ch = chunks[scale_chunks[blockIdx.x]];
    const DevTensor td = tensors[ch.tensor];
    constexpr uint32_t E = kChunkBytes / 4;
    const uint64_t c0 = uint64_t(ch.chunk_idx) * E;
    const uint32_t n_c = uint32_t(umin64(E, td.numel - c0));
    const DevPiece* pc = pieces + ch.first_piece;
    const uint32_t lane = threadIdx.x & 63u;
    if ((ch.n_pieces & kPiecesMask) == 1 && (n_c & 3u) == 0) {
        // one piece: each lane compares four consecutive scales with two
        // 128-bit loads; a wave covers 256 scales, four flag words, whose
        // bits come from four ballots (scale 4l + i is bit i of lane l's
        // nibble) spread so that lane l's nibble lands at bits 4l .. 4l + 3
        const uint64_t so = reinterpret_cast<uint64_t>(old_sh[pc[0].shard]) + (pc[0].shard_elem_off - pc[0].canon_start) * 4;
        const uint64_t sn = reinterpret_cast<uint64_t>(new_sh[pc[0].shard]) + (pc[0].shard_elem_off - pc[0].canon_start) * 4;
        if (((so | sn) & 15u) == 0) {
            auto spread4 = [](uint64_t x) {   // bit i of a 16-bit value to bit 4i
                x &= 0xFFFFu;
                x = (x | (x << 24)) & 0x000000FF000000FFull;
                x = (x | (x << 12)) & 0x000F000F000F000Full;
                x = (x | (x << 6)) & 0x0303030303030303ull;
                x = (x | (x << 3)) & 0x1111111111111111ull;
                return x;
            };
            for (uint32_t e0 = (threadIdx.x & ~63u) * 4; e0 < n_c; e0 += 1024) {
                const uint32_t e = e0 + 4 * lane;
                uint32_t nib = 0;
                if (e < n_c) {
                    const v4u o = __builtin_nontemporal_load(reinterpret_cast<gv4p>(so + uint64_t(e) * 4));
                    const v4u n = __builtin_nontemporal_load(reinterpret_cast<gv4p>(sn + uint64_t(e) * 4));
                    nib = uint32_t(o.x != n.x) | (uint32_t(o.y != n.y) << 1) | (uint32_t(o.z != n.z) << 2) |
                          (uint32_t(o.w != n.w) << 3);
                }
                const uint64_t m0 = __ballot(nib & 1u), m1 = __ballot(nib & 2u), m2 = __ballot(nib & 4u),
                               m3 = __ballot(nib & 8u);
                if (lane < 4 && e0 + 64 * lane < n_c) {
                    const uint32_t sh = 16 * lane;
                    flags[(td.scale_bit_off + c0 + e0 + 64 * lane) >> 6] =
                        spread4(m0 >> sh) | (spread4(m1 >> sh) << 1) | (spread4(m2 >> sh) << 2) |
                        (spread4(m3 >> sh) << 3);
                }
            }
            return;
        }
    }
    for (uint32_t e0 = (threadIdx.x & ~63u); e0 < n_c; e0 += 256) {
        const uint32_t e = e0 + lane;
        bool changed = false;
        if (e < n_c) {
            const uint32_t p = find_piece(pc, ch.n_pieces & kPiecesMask, e);
            const uint64_t off = (pc[p].shard_elem_off + (e - pc[p].canon_start)) * 4;
            changed = *reinterpret_cast<const uint32_t*>(old_sh[pc[p].shard] + off) !=
                      *reinterpret_cast<const uint32_t*>(new_sh[pc[p].shard] + off);
        }
        const uint64_t m = __ballot(changed);
        if (lane == 0) flags[(td.scale_bit_off + c0 + e0) >> 6] = m;
    }
}

// Stream header and encode result from the totals the fix-up stored.
// Partial retry: from a DELTA stream's directory and the receiver's applied
// flags, set the wanted bit of every chunk holding a record whose flag is 0.
// An entry that names no chunk of the plan sets the bad-directory counter.
__global__ __launch_bounds__(256) void retry_need_kernel(const uint8_t* dir, const uint8_t* flags, uint64_t n,
                                                         const DevTensor* tensors, uint32_t n_tensors,
                                                         uint64_t* need, uint32_t* counter) {
    for (uint64_t r = blockIdx.x * uint64_t(blockDim.x) + threadIdx.x; r < n;
         r += uint64_t(gridDim.x) * blockDim.x) {
        const uint2 tc = *reinterpret_cast<const uint2*>(dir + r * DCR_DIRENT_BYTES);
        if (tc.x >= n_tensors || tc.y >= tensors[tc.x].n_chunks) {
            atomicOr(counter + kCtrBad, 1u);
            continue;
        }
        if (flags[r]) continue;
        const uint32_t chunk = tensors[tc.x].first_chunk + tc.y;
        atomicOr(reinterpret_cast<unsigned long long*>(need + (chunk >> 6)), 1ull << (chunk & 63u));
    }
}

__device__ __forceinline__ void put_header(uint4* h, uint32_t mode, uint64_t base_v, uint64_t new_v, uint64_t fp,
                                           uint64_t nrec, uint64_t pbytes) {
    h[0] = make_uint4(DCR_MAGIC, DCR_FORMAT_VERSION | (mode << 16), DCR_CHUNK_BYTES, 0u);
    h[1] = make_uint4(uint32_t(base_v), uint32_t(base_v >> 32), uint32_t(new_v), uint32_t(new_v >> 32));
    h[2] = make_uint4(uint32_t(fp), uint32_t(fp >> 32), uint32_t(nrec), uint32_t(nrec >> 32));
    h[3] = make_uint4(uint32_t(pbytes), uint32_t(pbytes >> 32), 0u, 0u);
}

__global__ void encode_finalize_kernel(const uint32_t* counter, uint32_t mode, uint64_t base_v, uint64_t new_v,
                                       uint64_t fp, uint64_t dir_cap, uint64_t payload_cap, uint8_t* header,
                                       dcr_encode_result* res) {
    if (threadIdx.x != 0) return;
    const bool bad = counter[kCtrBad] != 0;   // partial retry given a directory naming no chunk
    const uint64_t v = bad ? 0 : *reinterpret_cast<const uint64_t*>(counter + kCtrTotal);
    const uint64_t nrec = v >> kRecShift, pbytes = (v & kP16Mask) << 4;
    const bool fits = nrec * DCR_DIRENT_BYTES <= dir_cap && pbytes <= payload_cap;
    put_header(reinterpret_cast<uint4*>(header), mode, base_v, new_v, fp, nrec, pbytes);
    const uint64_t changed = *reinterpret_cast<const uint64_t*>(counter + kCtrChanged);
    uint4* r = reinterpret_cast<uint4*>(res);
    r[0] = make_uint4(uint32_t(nrec), uint32_t(nrec >> 32), uint32_t(pbytes), uint32_t(pbytes >> 32));
    const int32_t st = bad ? DCR_E_FORMAT : (fits ? DCR_OK : DCR_E_CAPACITY);
    r[1] = make_uint4(uint32_t(changed), uint32_t(changed >> 32), uint32_t(st), counter[kRedoCtrOff / 4]);
}

// Ready watermark of a sliced encode: after slice k's fix-up blocks (the last
// being `last_blk`, or none when the plan has no tiles) the records before
// the slice's end are final.  Writes the header of the stream cut there into
// prefix slot k of the caller's host-visible region, then raises the count of
// published slices with a system-scope release, so that a host thread which
// reads the count also sees the header and, through the kernel boundary after
// the fix-up, the records.  A stream that does not fit its buffers, or a bad
// partial-retry directory, sets the region's status instead and publishes
// nothing more (both conditions, once true, stay true for every later slice).
__global__ void publish_kernel(const uint64_t* fix_status, uint32_t last_blk, const uint32_t* counter,
                               uint32_t mode, uint64_t base_v, uint64_t new_v, uint64_t fp, uint64_t dir_cap,
                               uint64_t payload_cap, uint8_t* ready, uint32_t k) {
    if (threadIdx.x != 0) return;
    const bool bad = counter[kCtrBad] != 0;
    const uint64_t v = last_blk == UINT32_MAX ? 0 : ld_status(fix_status + last_blk) >> kValShift;
    const uint64_t nrec = v >> kRecShift, pbytes = (v & kP16Mask) << 4;
    const bool fits = nrec * DCR_DIRENT_BYTES <= dir_cap && pbytes <= payload_cap;
    if (bad || !fits) {
        __hip_atomic_store(reinterpret_cast<int32_t*>(ready + 8), int32_t(bad ? DCR_E_FORMAT : DCR_E_CAPACITY),
                           __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
        return;
    }
    put_header(reinterpret_cast<uint4*>(ready + 64 + 64 * uint64_t(k)), mode, base_v, new_v, fp, nrec, pbytes);
    __hip_atomic_store(reinterpret_cast<uint64_t*>(ready), uint64_t(k) + 1u, __ATOMIC_RELEASE,
                       __HIP_MEMORY_SCOPE_SYSTEM);
}

__global__ void fill_u64_kernel(uint64_t* p, uint64_t n, uint64_t v) {
    for (uint64_t i = blockIdx.x * uint64_t(blockDim.x) + threadIdx.x; i < n; i += uint64_t(gridDim.x) * blockDim.x)
        p[i] = v;
}

// ------------------------------------------------------------------- apply

struct ApplyArgs {
    const DevTensor* tensors;
    uint8_t* const* canon;
    const uint8_t* dir;
    const uint8_t* payload;
    uint8_t* flags;
    dcr_apply_result* result;
    uint32_t* big_list;      // records (relative to first) deferred to the large-record kernel
    uint32_t* big_count;
    uint64_t payload_bytes;
    uint64_t first;
    uint32_t n_tensors;
    uint32_t retry;          // 1: overwrite retry (ignore flags, OW records only)
    // receiver layout: the records' chunks are written into shards through
    // the plan's pieces instead of into canonical tensors
    const DevChunk* rchunks;
    const DevPiece* rpieces;
    uint8_t* const* rshards;
    uint32_t sharded;
};

struct ApplyShared {
    alignas(16) uint8_t stage[kStageBytes];
    uint32_t pres_pre[1024];        // SPARSE: set presence bits before each 32-bit word
    uint64_t scan[2 * (kThreads / 64) + 1];
    uint32_t ent[8];                // the directory entry
    uint32_t state;                 // 0 invalid, 1 skip, 2 apply
    uint32_t n_c;                   // elements of the record's chunk
    uint32_t bad;                   // content check failed
    // receiver layout: the chunk's pieces (direct chunks: start element and
    // address of each piece, in LDS)
    uint32_t mfirst, mnp, mdirect;
    uint32_t mstart[kMaxCachedPieces];
    uint64_t maddr[kMaxCachedPieces];
};

__device__ __forceinline__ uint32_t rec_bytes(uint32_t n_c, uint32_t w, uint32_t kind, uint32_t K, uint32_t hm,
                                              uint32_t H, uint32_t layout) {
    uint32_t sz = (layout == DCR_LAYOUT_LIST ? dpad16(2 * K) : dpad16((n_c + 7) / 8)) + dpad16(K);
    if (w == 2 && kind == DCR_KIND_XOR) {
        if (hm == DCR_HI_SPARSE) sz += dpad16((K + 7) / 8) + dpad16(H);
        else if (hm == DCR_HI_DENSE) sz += dpad16(K);
    } else if (w == 2) sz += dpad16(K);
    else if (w == 4) sz += 3 * dpad16(K);
    return sz;
}

// Structural check of one directory entry (thread 0).
__device__ __forceinline__ bool entry_ok(const ApplyArgs& a, const uint32_t (&e)[8], uint32_t& n_c_out) {
    const uint32_t t = e[0], c = e[1], K = e[2];
    const uint32_t kind = e[3] & 0xFF, hm = (e[3] >> 8) & 0xFF, w = (e[3] >> 16) & 0xFF, z = e[3] >> 24;
    const uint64_t off = uint64_t(e[4]) | (uint64_t(e[5]) << 32);
    const uint32_t sz = e[6], H = e[7];
    if (t >= a.n_tensors || z > DCR_LAYOUT_LIST) return false;
    const DevTensor td = a.tensors[t];
    if (w != td.w || c >= td.n_chunks) return false;
    const uint64_t E = kChunkBytes / w;
    const uint32_t n_c = uint32_t(umin64(E, td.numel - uint64_t(c) * E));
    if (K == 0 || K > n_c || kind > DCR_KIND_OW) return false;
    if (a.retry && kind != DCR_KIND_OW) return false;
    if (kind == DCR_KIND_XOR && w == 4) return false;
    if (w == 1) {
        if (hm != DCR_HI_NONE || H != 0) return false;
    } else if (kind == DCR_KIND_OW) {
        if (hm != DCR_HI_DENSE || H != K) return false;
    } else if (hm == DCR_HI_NONE) {
        if (H != 0) return false;
    } else if (hm == DCR_HI_SPARSE) {
        if (H == 0 || H > K || !(dpad16((K + 7) / 8) + dpad16(H) < dpad16(K))) return false;
    } else if (hm == DCR_HI_DENSE) {
        if (H != K) return false;
    } else {
        return false;
    }
    if (sz != rec_bytes(n_c, w, kind, K, hm, H, z)) return false;
    if ((off & 15u) != 0 || off > a.payload_bytes || sz > a.payload_bytes - off) return false;
    n_c_out = n_c;
    return true;
}

// Receiver layout, thread 0: the record's chunk in the receiver plan.
template <class Sh>
__device__ __forceinline__ void map_chunk(const ApplyArgs& a, Sh& S, uint32_t t, uint32_t c) {
    if (!a.sharded) return;
    const DevChunk ch = a.rchunks[a.tensors[t].first_chunk + c];
    S.mfirst = ch.first_piece;
    S.mnp = ch.n_pieces & kPiecesMask;
    S.mdirect = (ch.n_pieces & kChunkDirect) ? 1u : 0u;
}

// Receiver layout, all threads before a barrier: a direct chunk's piece
// table in LDS.
template <int W, class Sh>
__device__ __forceinline__ void map_table(const ApplyArgs& a, Sh& S) {
    if (!a.sharded || !S.mdirect || threadIdx.x >= S.mnp) return;
    const DevPiece p = a.rpieces[S.mfirst + threadIdx.x];
    S.mstart[threadIdx.x] = p.canon_start;
    S.maddr[threadIdx.x] = reinterpret_cast<uint64_t>(a.rshards[p.shard]) + p.shard_elem_off * W;
}

// Address of the 16-byte group starting at chunk element e0: in the
// canonical chunk at dst, or in a direct receiver chunk (every group inside
// one piece, 16-byte aligned); NULL for other receiver chunks, whose
// elements are mapped one by one.
template <int W, class Sh>
__device__ __forceinline__ uint8_t* group_ptr(const ApplyArgs& a, const Sh& S, uint8_t* dst, uint32_t e0) {
    if (!a.sharded) return dst + uint64_t(e0) * W;
    if (!S.mdirect) return nullptr;
    uint32_t l = 0, h = S.mnp;
    while (h - l > 1) {
        const uint32_t m = (l + h) >> 1;
        if (S.mstart[m] <= e0) l = m;
        else h = m;
    }
    return reinterpret_cast<uint8_t*>(S.maddr[l] + uint64_t(e0 - S.mstart[l]) * W);
}

// Address of chunk element e of a receiver chunk (its pieces in global
// memory, found by binary search on their first element).
template <int W, class Sh>
__device__ __forceinline__ uint8_t* elem_ptr(const ApplyArgs& a, const Sh& S, uint32_t e) {
    const DevPiece* pc = a.rpieces + S.mfirst;
    uint32_t l = 0, h = S.mnp;
    while (h - l > 1) {
        const uint32_t m = (l + h) >> 1;
        if (pc[m].canon_start <= e) l = m;
        else h = m;
    }
    const DevPiece p = pc[l];
    return a.rshards[p.shard] + (p.shard_elem_off + (e - p.canon_start)) * W;
}

template <int W>
__device__ void apply_record(const ApplyArgs& a, ApplyShared& S, uint64_t r, uint32_t n_c) {
    constexpr uint32_t V = 16 / W;
    constexpr uint32_t E = kChunkBytes / W;
    const uint32_t tid = threadIdx.x;
    const uint32_t t = S.ent[0], c = S.ent[1], K = S.ent[2];
    const uint32_t kind = S.ent[3] & 0xFF, hm = (S.ent[3] >> 8) & 0xFF;
    const uint64_t off = uint64_t(S.ent[4]) | (uint64_t(S.ent[5]) << 32);
    const uint32_t sz = S.ent[6], H = S.ent[7];
    const uint32_t bm = dpad16((n_c + 7) / 8);
    const uint32_t lo = bm;
    const uint32_t pres = lo + dpad16(K);
    const uint32_t hi = hm == DCR_HI_SPARSE ? pres + dpad16((K + 7) / 8) : pres;

    // stage the record
    const uint4* src = reinterpret_cast<const uint4*>(a.payload + off);
    for (uint32_t q = tid; q < sz / 16; q += kThreads) reinterpret_cast<uint4*>(S.stage)[q] = src[q];
    if (tid == 0) S.bad = 0;
    map_table<W>(a, S);
    __syncthreads();

    // bitmap bits per 16-byte group; nothing may be set at or past n_c
    uint32_t bits[kVecsPerThread];
    uint64_t cnt[1] = {0};
    bool bad = false;
#pragma unroll
    for (uint32_t k = 0; k < kVecsPerThread; k++) {
        const uint32_t g = tid + k * kThreads;
        uint32_t b = 0;
        if (g * V < bm * 8) {   // the group's bits lie inside the padded bitmap
            if constexpr (W == 2) b = S.stage[g];
            else if constexpr (W == 1) b = reinterpret_cast<const uint16_t*>(S.stage)[g];
            else b = (S.stage[g / 2] >> (4 * (g & 1))) & 0xFu;
        }
        const uint32_t first = g * V;
        const uint32_t valid = first >= n_c ? 0u : (n_c - first >= V ? (1u << V) - 1u : (1u << (n_c - first)) - 1u);
        if (b & ~valid) bad = true;
        bits[k] = b & valid;
        cnt[0] |= uint64_t(__popc(bits[k])) << (16 * k);
    }
    // SPARSE: presence bits, popcount H, nothing at or past K; word prefix counts
    uint64_t pc1[1] = {0};
    uint32_t pword = 0;
    const uint32_t n_pw = dpad16((K + 7) / 8) / 4;
    if (hm == DCR_HI_SPARSE && tid < n_pw) {
        pword = reinterpret_cast<const uint32_t*>(S.stage + pres)[tid];
        const uint32_t b0 = tid * 32;
        const uint32_t vmask = b0 >= K ? 0u : (K - b0 >= 32 ? 0xFFFFFFFFu : ((1u << (K - b0)) - 1u));
        if (pword & ~vmask) bad = true;
        pc1[0] = __popc(pword);
    }
    uint64_t tot[1], ptot[1];
    block_excl_scan<1>(cnt, tot, S.scan);
    if (hm == DCR_HI_SPARSE) {
        block_excl_scan<1>(pc1, ptot, S.scan);
        if (tid < n_pw) S.pres_pre[tid] = uint32_t(pc1[0]);
        if (tid == 0 && ptot[0] != H) bad = true;
    }
    uint32_t total = 0, base[kVecsPerThread];
#pragma unroll
    for (uint32_t k = 0; k < kVecsPerThread; k++) {
        base[k] = total + field16(cnt[0], k);
        total += field16(tot[0], k);
    }
    if (tid == 0 && total != K) bad = true;
    if (bad) atomicOr(&S.bad, 1u);
    __syncthreads();
    if (S.bad) return;   // refused before any write

    // read-modify-write of every touched 16-byte group; the group's new words
    // are assembled in two 64-bit values by a set-bit loop with dynamic shifts
    uint8_t* dst = a.sharded ? nullptr : a.canon[t] + uint64_t(c) * E * W;
    const uint32_t* pw32 = reinterpret_cast<const uint32_t*>(S.stage + pres);
    const uint32_t pk = dpad16(K);
    const bool is_xor = kind == DCR_KIND_XOR;
#pragma unroll
    for (uint32_t k = 0; k < kVecsPerThread; k++) {
        uint32_t b = bits[k];
        if (!b) continue;
        const uint32_t g = tid + k * kThreads;
        uint64_t val0 = 0, val1 = 0, msk0 = 0, msk1 = 0;
        uint32_t j = base[k];
        const uint32_t bcopy = b;
        while (b) {
            const uint32_t i = uint32_t(__ffs(b) - 1);
            b &= b - 1;
            uint32_t v = S.stage[lo + j];
            if constexpr (W == 2) {
                if (!is_xor || hm == DCR_HI_DENSE) {
                    v |= uint32_t(S.stage[hi + j]) << 8;
                } else if (hm == DCR_HI_SPARSE) {
                    const uint32_t pwj = pw32[j >> 5];
                    if ((pwj >> (j & 31)) & 1u) {
                        const uint32_t rank = S.pres_pre[j >> 5] + __popc(pwj & ((1u << (j & 31)) - 1u));
                        v |= uint32_t(S.stage[hi + rank]) << 8;
                    }
                }
            } else if constexpr (W == 4) {
                v |= uint32_t(S.stage[lo + pk + j]) << 8;
                v |= uint32_t(S.stage[lo + 2 * pk + j]) << 16;
                v |= uint32_t(S.stage[lo + 3 * pk + j]) << 24;
            }
            constexpr uint32_t EB = 8 * W;                   // element bits
            constexpr uint64_t EM = (W == 4) ? 0xFFFFFFFFull : ((1ull << EB) - 1);
            const uint32_t bitpos = i * EB;                  // 0 .. 127
            const uint32_t sh = bitpos & 63;
            if (bitpos < 64) { val0 |= uint64_t(v) << sh; msk0 |= EM << sh; }
            else { val1 |= uint64_t(v) << sh; msk1 |= EM << sh; }
            j++;
        }
        uint8_t* gp = group_ptr<W>(a, S, dst, g * V);
        if (gp && (g + 1) * V <= n_c) {
            v4u w4 = *reinterpret_cast<const v4u*>(gp);
            uint64_t q0 = uint64_t(w4.x) | (uint64_t(w4.y) << 32);
            uint64_t q1 = uint64_t(w4.z) | (uint64_t(w4.w) << 32);
            q0 = is_xor ? (q0 ^ val0) : ((q0 & ~msk0) | val0);
            q1 = is_xor ? (q1 ^ val1) : ((q1 & ~msk1) | val1);
            v4u r4;
            r4.x = uint32_t(q0); r4.y = uint32_t(q0 >> 32); r4.z = uint32_t(q1); r4.w = uint32_t(q1 >> 32);
            *reinterpret_cast<v4u*>(gp) = r4;
        } else {
            // tail group of a tensor, or a receiver chunk whose groups are not whole in one piece: element accesses only, inside the tensor
            uint32_t bb = bcopy;
            while (bb) {
                const uint32_t i = uint32_t(__ffs(bb) - 1);
                bb &= bb - 1;
                if (g * V + i >= n_c) break;
                const uint32_t bitpos = i * 8 * W;
                const uint32_t v = uint32_t(((bitpos < 64) ? val0 : val1) >> (bitpos & 63));
                uint8_t* ep = gp ? gp + i * W : elem_ptr<W>(a, S, g * V + i);
                if constexpr (W == 1) { *ep = is_xor ? uint8_t(*ep ^ v) : uint8_t(v); }
                else if constexpr (W == 2) {
                    uint16_t* p = reinterpret_cast<uint16_t*>(ep);
                    *p = is_xor ? uint16_t(*p ^ v) : uint16_t(v);
                } else {
                    uint32_t* p = reinterpret_cast<uint32_t*>(ep);
                    *p = is_xor ? (*p ^ v) : v;
                }
            }
        }
    }
    __syncthreads();
    if (tid == 0) {
        // The flag becomes visible with the record's writes at kernel
        // completion (stream order); no cross-agent ordering is promised
        // while the kernel runs, so no device-wide fence is paid per record.
        if (!a.retry) a.flags[r] = 1;
    }
}

// One record with the large-record path: state already decided by the
// caller (entry checked, dedup flag read).  Counts only refusals and skips;
// the applied count is derived at the end.
__device__ __forceinline__ void apply_one(const ApplyArgs& a, ApplyShared& S, uint64_t r) {
    uint32_t n_c = 0;
    if (threadIdx.x == 0) {
        const uint4* de = reinterpret_cast<const uint4*>(a.dir + r * DCR_DIRENT_BYTES);
        const uint4 e0 = de[0], e1 = de[1];
        uint32_t e[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
        for (int i = 0; i < 8; i++) S.ent[i] = e[i];
        uint32_t st;
        // an index-list record always fits the small-record stage (its list
        // is smaller than the bitmap): one here is malformed
        if (!entry_ok(a, e, n_c) || (e[3] >> 24) != DCR_LAYOUT_BITMAP) st = 0;
        else if (!a.retry && a.flags[r]) st = 1;
        else st = 2;
        if (st == 2) map_chunk(a, S, e[0], e[1]);
        S.state = st;
        S.n_c = n_c;
    }
    __syncthreads();
    const uint32_t st = S.state;
    n_c = S.n_c;
    if (st == 1) {
        if (threadIdx.x == 0) atomicAdd(reinterpret_cast<unsigned long long*>(&a.result->n_skipped), 1ull);
        return;
    }
    if (st == 2) {
        const uint32_t w = (S.ent[3] >> 16) & 0xFF;
        if (w == 2) apply_record<2>(a, S, r, n_c);
        else if (w == 1) apply_record<1>(a, S, r, n_c);
        else apply_record<4>(a, S, r, n_c);
        if (!S.bad) return;
    }
    if (threadIdx.x == 0) {
        atomicAdd(reinterpret_cast<unsigned long long*>(&a.result->n_invalid), 1ull);
        atomicMin(reinterpret_cast<unsigned long long*>(&a.result->first_invalid), (unsigned long long)r);
    }
}

// Large-record apply, one workgroup per record of [first, first + n).
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(8, 8))) void apply_kernel(ApplyArgs a) {
    __shared__ ApplyShared S;
    apply_one(a, S, a.first + blockIdx.x);
}

// Large-record apply over the records the small-record kernel deferred: a
// persistent grid looping over the list.
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(8, 8))) void apply_big_kernel(ApplyArgs a) {
    __shared__ ApplyShared S;
    const uint32_t n = *a.big_count;
    for (uint32_t i = blockIdx.x; i < n; i += gridDim.x) {
        apply_one(a, S, a.first + a.big_list[i]);
        __syncthreads();
    }
}

// Small-record apply: a workgroup of kSmallThreads per record, the record
// staged in a kSmallStage LDS buffer, so that many records per compute unit
// are in flight.  Thread t owns the 16 consecutive 16-byte groups starting
// at group 16t (its bitmap bits are contiguous, so one scan of per-thread
// change counts ranks every change).  Records that do not fit go to the
// large-record kernel.
constexpr uint32_t kLinesPerChunk = kChunkBytes / 128;
struct SmallShared {
    alignas(16) uint8_t stage[kSmallStage];
    uint32_t pres_pre[kSmallThreads];   // SPARSE: set presence bits before each 32-bit word
    uint32_t jpre[kSmallThreads];       // line mode: changes before each thread's bitmap slice
    uint32_t jpre2[kSmallThreads];      // ... of a fused pair's overwrite record
    uint8_t whole[kLinesPerChunk];      // line mode: lines that may be read and written whole
    uint8_t other[kLinesPerChunk];      // line mode beside another record: lines that record marks
    uint64_t scan[kSmallThreads / 64];
    uint32_t ent[8];
    uint32_t ent2[8];                   // fused pair: the overwrite record's entry
    uint32_t state;                     // 0 invalid, 1 skip, 2 apply, 3 deferred, 4 left to the pair's XOR record
    uint32_t n_c;
    uint32_t bad;
    uint32_t bad2;                      // fused pair: the overwrite record is malformed
    uint32_t fused;                     // 1: the overwrite record at rec + 1 is applied here too
    uint32_t pskip;                     // 1: the other record of this record's pair is skipped (flagged)
    uint64_t rec;                       // the record this workgroup applies
    uint32_t solo;                      // 1: no other record of this call names the same chunk;
                                        // 2: one other does, a bitmap record at sib_off (below)
    uint64_t sib_off;                   // payload offset of that other record
    uint64_t dst;                       // canonical layout: the chunk's first byte
    uint32_t sib;                       // line mode beside it (its lines flagged in `other`)
    uint32_t mfirst, mnp, mdirect;      // receiver layout (as in ApplyShared)
    uint32_t mstart[kMaxCachedPieces];
    uint64_t maddr[kMaxCachedPieces];
};

// Exclusive scan of one count per thread over a kSmallThreads workgroup (the
// workgroup's sum stays below 2^32: changes of one chunk).
__device__ __forceinline__ uint64_t small_excl_scan(uint64_t v, uint64_t& total, uint64_t* sh) {
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    const uint64_t inc = wave_incl_scan_halves(v);
    if (lane == 63) sh[wave] = inc;
    __syncthreads();
    uint64_t pre = 0, tot = 0;
#pragma unroll
    for (uint32_t w = 0; w < kSmallThreads / 64; w++) {
        pre += w < wave ? sh[w] : 0;
        tot += sh[w];
    }
    __syncthreads();
    total = tot;
    return pre + inc - v;
}

// The new bits (overwrite) or XOR mask of the changed elements of one
// 16-byte group, b = the group's change bits, j = the record index of its
// first change (advanced past the group): packed into a 128-bit value with
// the mask of the elements it covers.
template <int W>
__device__ __forceinline__ void group_value(const SmallShared& S, uint32_t b, uint32_t& j, uint32_t lo, uint32_t hi,
                                            uint32_t pres, uint32_t pk, uint32_t hm, bool is_xor, uint64_t& val0,
                                            uint64_t& val1, uint64_t& msk0, uint64_t& msk1) {
    const uint32_t* pw32 = reinterpret_cast<const uint32_t*>(S.stage + pres);
    val0 = val1 = msk0 = msk1 = 0;
    while (b) {
        const uint32_t i = uint32_t(__ffs(b) - 1);
        b &= b - 1;
        uint32_t v = S.stage[lo + j];
        if constexpr (W == 2) {
            if (!is_xor || hm == DCR_HI_DENSE) {
                v |= uint32_t(S.stage[hi + j]) << 8;
            } else if (hm == DCR_HI_SPARSE) {
                const uint32_t pwj = pw32[j >> 5];
                if ((pwj >> (j & 31)) & 1u) {
                    const uint32_t rank = S.pres_pre[j >> 5] + __popc(pwj & ((1u << (j & 31)) - 1u));
                    v |= uint32_t(S.stage[hi + rank]) << 8;
                }
            }
        } else if constexpr (W == 4) {
            v |= uint32_t(S.stage[lo + pk + j]) << 8;
            v |= uint32_t(S.stage[lo + 2 * pk + j]) << 16;
            v |= uint32_t(S.stage[lo + 3 * pk + j]) << 24;
        }
        constexpr uint32_t EB = 8 * W;
        constexpr uint64_t EM = (W == 4) ? 0xFFFFFFFFull : ((1ull << EB) - 1);
        const uint32_t bitpos = i * EB;
        const uint32_t sh = bitpos & 63;
        if (bitpos < 64) { val0 |= uint64_t(v) << sh; msk0 |= EM << sh; }
        else { val1 |= uint64_t(v) << sh; msk1 |= EM << sh; }
        j++;
    }
}

// One patched 16-byte group (XOR or merge under the mask).
__device__ __forceinline__ v4u patch16(v4u w4, bool is_xor, uint64_t val0, uint64_t val1, uint64_t msk0,
                                       uint64_t msk1) {
    uint64_t q0 = uint64_t(w4.x) | (uint64_t(w4.y) << 32);
    uint64_t q1 = uint64_t(w4.z) | (uint64_t(w4.w) << 32);
    q0 = is_xor ? (q0 ^ val0) : ((q0 & ~msk0) | val0);
    q1 = is_xor ? (q1 ^ val1) : ((q1 & ~msk1) | val1);
    v4u r4;
    r4.x = uint32_t(q0); r4.y = uint32_t(q0 >> 32); r4.z = uint32_t(q1); r4.w = uint32_t(q1 >> 32);
    return r4;
}

// Element-wise patch of the changed elements (bits b) of group g of a
// canonical chunk at dst, those below n_c only.
template <int W>
__device__ __forceinline__ void patch_elems(uint8_t* dst, uint32_t g, uint32_t b, uint32_t n_c, bool is_xor,
                                            uint64_t val0, uint64_t val1) {
    constexpr uint32_t V = 16 / W;
    while (b) {
        const uint32_t i = uint32_t(__ffs(b) - 1);
        b &= b - 1;
        if (g * V + i >= n_c) break;
        const uint32_t bitpos = i * 8 * W;
        const uint32_t v = uint32_t(((bitpos < 64) ? val0 : val1) >> (bitpos & 63));
        uint8_t* ep = dst + (uint64_t(g) * V + i) * W;
        if constexpr (W == 1) { *ep = is_xor ? uint8_t(*ep ^ v) : uint8_t(v); }
        else if constexpr (W == 2) {
            uint16_t* p = reinterpret_cast<uint16_t*>(ep);
            *p = is_xor ? uint16_t(*p ^ v) : uint16_t(v);
        } else {
            uint32_t* p = reinterpret_cast<uint32_t*>(ep);
            *p = is_xor ? (*p ^ v) : v;
        }
    }
}

// Line mode of the small-record apply (canonical chunk at dst, 128-byte
// aligned): in iteration k lane l takes group k * kSmallThreads + l, so each
// wave covers 64 consecutive groups; every 128-byte line that holds a change
// of the record and lies wholly inside the chunk's elements is read and
// written whole by its 8 lanes (unchanged groups written back as read), which
// the memory takes as full-line writes.  Groups of a line that crosses the
// chunk's end are patched on their own (whole groups with 128-bit accesses,
// the ragged one element by element).  Needs S.jpre: the changes before each
// thread's 16-group bitmap slice, and the record's change bitmap in the
// stage at byte bmo (0 for a bitmap record; a list record's bitmap is
// rebuilt past the record).  pair: a fused pair, whose overwrite record is
// staged at bmo2 (bitmap, then its byte planes from lo2, pk2 apart) with its
// slice prefixes in S.jpre2; a line touched by either record is written
// whole, each group patched from the record that marks it.
template <int W>
__device__ __forceinline__ void apply_lines(const SmallShared& S, uint8_t* dst, uint32_t n_c, uint32_t lo,
                                            uint32_t hi, uint32_t pres, uint32_t pk, uint32_t hm, bool is_xor,
                                            uint32_t bmo, bool pair, uint32_t bmo2, uint32_t lo2, uint32_t pk2,
                                            uint32_t hm2) {
    constexpr uint32_t V = 16 / W;                        // change bits per group
    constexpr uint32_t GT = kVecsPerChunk / kSmallThreads;  // groups per bitmap slice (16)
    constexpr uint32_t BB = GT * V / 8;                   // bitmap bytes per slice
    constexpr uint32_t LG = 8;                            // groups per 128-byte line
    constexpr uint32_t KB = 4;                            // groups per lane loaded before patching
    constexpr uint32_t GM = (V == 16) ? 0xFFFFu : ((1u << V) - 1u);
    const uint32_t tid = threadIdx.x;
    const uint32_t n_groups = (n_c + V - 1) / V;
    // a line's change bits in the bitmap at stage offset b (bits past n_c
    // were refused, so they are zero); the group's own bits in gbits
    auto line_bits = [&](uint32_t b, uint32_t L, uint32_t q, uint32_t& gbits) {
        bool touched;
        if constexpr (W == 2) {
            const uint64_t lb = *reinterpret_cast<const uint64_t*>(S.stage + b + 8 * L);
            touched = lb != 0;
            gbits = uint32_t(lb >> (8 * q)) & GM;
        } else if constexpr (W == 1) {
            const uint4 lb = *reinterpret_cast<const uint4*>(S.stage + b + 16 * L);
            touched = (lb.x | lb.y | lb.z | lb.w) != 0;
            const uint32_t wv = (q & 4u) ? ((q & 2u) ? lb.w : lb.z) : ((q & 2u) ? lb.y : lb.x);
            gbits = (wv >> (16 * (q & 1u))) & GM;
        } else {
            const uint32_t lb = *reinterpret_cast<const uint32_t*>(S.stage + b + 4 * L);
            touched = lb != 0;
            gbits = (lb >> (4 * q)) & GM;
        }
        return touched;
    };
    // record index of group g's first change: the changes before its slice
    // plus those of the slice's earlier groups
    auto first_index = [&](uint32_t b, uint32_t pre, uint32_t g) {
        const uint32_t sl = g / GT, nb = (g % GT) * V;
        uint32_t j = pre;
#pragma unroll
        for (uint32_t i = 0; i < BB / 4; i++) {
            const uint32_t wd = *reinterpret_cast<const uint32_t*>(S.stage + b + sl * BB + 4 * i);
            const uint32_t m = nb >= 32 * (i + 1) ? 0xFFFFFFFFu : (nb <= 32 * i ? 0u : ((1u << (nb - 32 * i)) - 1u));
            j += __popc(wd & m);
        }
        return j;
    };
    for (uint32_t k0 = 0; k0 < GT; k0 += KB) {
        v4u v[KB];
        uint32_t gb[KB], st[KB];   // change bits; 0 skip, 1 whole line, 2 group alone
        uint32_t ob = 0;           // a fused pair: which of the KB groups are the overwrite record's
#pragma unroll
        for (uint32_t kk = 0; kk < KB; kk++) {
            const uint32_t g = (k0 + kk) * kSmallThreads + tid;
            const uint32_t L = g / LG, q = g % LG;
            uint32_t s_ = 0, b = 0;
            if (g < n_groups) {
                bool touched = line_bits(bmo, L, q, b);
                if (pair) {
                    // the pair's groups are disjoint: a group is the XOR
                    // record's, the overwrite record's or neither's
                    uint32_t b2;
                    touched |= line_bits(bmo2, L, q, b2);
                    if (b2) {
                        b = b2;
                        ob |= 1u << kk;
                    }
                }
                // a line that may not be written whole (the chunk's other
                // record marks it, or it passes the chunk's end): this
                // record's groups alone
                if (touched) s_ = S.whole[L] ? 1u : (b ? 2u : 0u);
            }
            st[kk] = s_;
            gb[kk] = b;
            if (s_ == 1) v[kk] = *reinterpret_cast<const v4u*>(dst + uint64_t(g) * 16);
        }
#pragma unroll
        for (uint32_t kk = 0; kk < KB; kk++) {
            if (!st[kk]) continue;
            const uint32_t g = (k0 + kk) * kSmallThreads + tid;
            const bool ow2 = (ob >> kk) & 1u;
            const bool x = ow2 ? false : is_xor;
            uint64_t val0 = 0, val1 = 0, msk0 = 0, msk1 = 0;
            if (gb[kk]) {
                if (ow2) {
                    uint32_t j = first_index(bmo2, S.jpre2[g / GT], g);
                    group_value<W>(S, gb[kk], j, lo2, lo2 + pk2, lo2 + pk2, pk2, hm2, false, val0, val1, msk0,
                                   msk1);
                } else {
                    uint32_t j = first_index(bmo, S.jpre[g / GT], g);
                    group_value<W>(S, gb[kk], j, lo, hi, pres, pk, hm, is_xor, val0, val1, msk0, msk1);
                }
            }
            uint8_t* gp = dst + uint64_t(g) * 16;
            if (st[kk] == 1) {
                *reinterpret_cast<v4u*>(gp) = gb[kk] ? patch16(v[kk], x, val0, val1, msk0, msk1) : v[kk];
            } else if ((g + 1) * V <= n_c) {
                *reinterpret_cast<v4u*>(gp) = patch16(*reinterpret_cast<const v4u*>(gp), x, val0, val1, msk0, msk1);
            } else {
                patch_elems<W>(dst, g, gb[kk], n_c, x, val0, val1);
            }
        }
    }
}

// A thread's slice of a staged bitmap (bytes [b0, b0 + 4 NW) of the bitmap
// at stage offset base, bm bytes long; bytes at or past bm are other
// sections: read as 0), as whole 64- / 128-bit LDS reads (word reads at
// this stride would collide on the banks).
template <uint32_t NW>
__device__ __forceinline__ void bitmap_slice(const SmallShared& S, uint32_t base, uint32_t b0, uint32_t bm,
                                             uint32_t (&raw)[NW]) {
    if constexpr (NW == 2) {
        const uint2 v = b0 < bm ? *reinterpret_cast<const uint2*>(S.stage + base + b0) : make_uint2(0, 0);
        raw[0] = v.x;
        raw[1] = v.y;
    } else {
#pragma unroll
        for (uint32_t h = 0; h < NW / 4; h++) {
            const uint4 v = b0 + 16 * h < bm ? *reinterpret_cast<const uint4*>(S.stage + base + b0 + 16 * h)
                                             : make_uint4(0, 0, 0, 0);
            raw[4 * h] = v.x;
            raw[4 * h + 1] = v.y;
            raw[4 * h + 2] = v.z;
            raw[4 * h + 3] = v.w;
        }
    }
}

// Nothing may be set at or past n_c: such bits make the record bad and are
// dropped.  Returns the slice's change count.
template <uint32_t NW>
__device__ __forceinline__ uint32_t checked_slice(uint32_t (&x)[NW], uint32_t b0, uint32_t n_c, bool& bad) {
    uint32_t cnt = 0;
#pragma unroll
    for (uint32_t i = 0; i < NW; i++) {
        const uint32_t e0 = (b0 + 4 * i) * 8;
        const uint32_t valid = e0 >= n_c ? 0u : (n_c - e0 >= 32 ? 0xFFFFFFFFu : ((1u << (n_c - e0)) - 1u));
        if (x[i] & ~valid) bad = true;
        x[i] &= valid;
        cnt += __popc(x[i]);
    }
    return cnt;
}

// Read-modify-write of every 16-byte group a thread's bitmap slice bw marks,
// in element order; j = the record index of the slice's first change.  The
// record's sections sit at stage offsets lo / pres / hi.
template <int W, uint32_t NW>
__device__ __forceinline__ void apply_groups(const ApplyArgs& a, const SmallShared& S, uint8_t* dst, uint32_t n_c,
                                             const uint32_t (&bw)[NW], uint32_t j, uint32_t lo, uint32_t hi,
                                             uint32_t pres, uint32_t pk, uint32_t hm, bool is_xor) {
    constexpr uint32_t V = 16 / W;
    constexpr uint32_t GT = kVecsPerChunk / kSmallThreads;
    constexpr uint32_t GPW = 32 / V;
    constexpr uint32_t GM = (V == 16) ? 0xFFFFu : ((1u << V) - 1u);
#pragma unroll
    for (uint32_t wi = 0; wi < NW; wi++) {
        uint32_t wv = bw[wi];
        while (wv) {
            const uint32_t gi = uint32_t(__ffs(wv) - 1) / V;
            uint32_t b = (wv >> (gi * V)) & GM;
            wv &= ~(GM << (gi * V));
            const uint32_t g = threadIdx.x * GT + wi * GPW + gi;
            uint64_t val0, val1, msk0, msk1;
            const uint32_t bcopy = b;
            group_value<W>(S, b, j, lo, hi, pres, pk, hm, is_xor, val0, val1, msk0, msk1);
            uint8_t* gp = group_ptr<W>(a, S, dst, g * V);
            if (gp && (g + 1) * V <= n_c) {
                *reinterpret_cast<v4u*>(gp) = patch16(*reinterpret_cast<const v4u*>(gp), is_xor, val0, val1, msk0,
                                                      msk1);
            } else {
                // tail group of a tensor, or a receiver chunk whose groups are not whole in one piece: element accesses only, inside the tensor
                uint32_t bb = bcopy;
                while (bb) {
                    const uint32_t i = uint32_t(__ffs(bb) - 1);
                    bb &= bb - 1;
                    if (g * V + i >= n_c) break;
                    const uint32_t bitpos = i * 8 * W;
                    const uint32_t v = uint32_t(((bitpos < 64) ? val0 : val1) >> (bitpos & 63));
                    uint8_t* ep = gp ? gp + i * W : elem_ptr<W>(a, S, g * V + i);
                    if constexpr (W == 1) { *ep = is_xor ? uint8_t(*ep ^ v) : uint8_t(v); }
                    else if constexpr (W == 2) {
                        uint16_t* p = reinterpret_cast<uint16_t*>(ep);
                        *p = is_xor ? uint16_t(*p ^ v) : uint16_t(v);
                    } else {
                        uint32_t* p = reinterpret_cast<uint32_t*>(ep);
                        *p = is_xor ? (*p ^ v) : v;
                    }
                }
            }
        }
    }
}

template <int W, bool PAIRS>
__device__ __forceinline__ void apply_small_record(const ApplyArgs& a, SmallShared& S, uint64_t r, uint32_t n_c) {
    constexpr uint32_t V = 16 / W;                        // elements (= bitmap bits) per group
    constexpr uint32_t GT = kVecsPerChunk / kSmallThreads;  // groups per thread (16)
    constexpr uint32_t BB = GT * V / 8;                   // bitmap bytes per thread (8, 16 or 32)
    constexpr uint32_t NW = BB / 4;                       // ... in 32-bit words
    const uint32_t tid = threadIdx.x;
    const uint32_t K = S.ent[2];
    const uint32_t kind = S.ent[3] & 0xFF, hm = (S.ent[3] >> 8) & 0xFF;
    const uint64_t off = uint64_t(S.ent[4]) | (uint64_t(S.ent[5]) << 32);
    const uint32_t sz = S.ent[6], H = S.ent[7];
    const uint32_t bm = dpad16((n_c + 7) / 8);
    const uint32_t layout = S.ent[3] >> 24;   // bitmap or index list (checked by entry_ok)
    const uint32_t lo = layout == DCR_LAYOUT_LIST ? dpad16(2 * K) : bm;
    const uint32_t pres = lo + dpad16(K);
    const uint32_t hi = hm == DCR_HI_SPARSE ? pres + dpad16((K + 7) / 8) : pres;

    // stage the record (and a fused pair's overwrite record right after it);
    // for line mode beside the chunk's other record, flag the lines that
    // record's bitmap marks (V bitmap bytes per line)
    const uint4* src = reinterpret_cast<const uint4*>(a.payload + off);
    for (uint32_t q = tid; q < sz / 16; q += kSmallThreads)   // read once: non-temporal
        reinterpret_cast<v4u*>(S.stage)[q] =
            __builtin_nontemporal_load(reinterpret_cast<gv4p>(reinterpret_cast<uintptr_t>(src)) + q);
    const uint32_t fused = PAIRS ? S.fused : 0u;
    if (fused) {
        const uint64_t off2 = uint64_t(S.ent2[4]) | (uint64_t(S.ent2[5]) << 32);
        const uint4* src2 = reinterpret_cast<const uint4*>(a.payload + off2);
        for (uint32_t q = tid; q < S.ent2[6] / 16; q += kSmallThreads)
            reinterpret_cast<v4u*>(S.stage + sz)[q] =
                __builtin_nontemporal_load(reinterpret_cast<gv4p>(reinterpret_cast<uintptr_t>(src2)) + q);
    }
    if (S.sib) {
        const uint4* ssrc = reinterpret_cast<const uint4*>(a.payload + S.sib_off);
        for (uint32_t q = tid; q < bm / 16; q += kSmallThreads) {
            const uint4 v = ssrc[q];
            if constexpr (W == 2) {
                S.other[2 * q] = (v.x | v.y) != 0;
                S.other[2 * q + 1] = (v.z | v.w) != 0;
            } else if constexpr (W == 1) {
                S.other[q] = (v.x | v.y | v.z | v.w) != 0;
            } else {
                S.other[4 * q] = v.x != 0;
                S.other[4 * q + 1] = v.y != 0;
                S.other[4 * q + 2] = v.z != 0;
                S.other[4 * q + 3] = v.w != 0;
            }
        }
    }
    if (tid == 0) S.bad = S.bad2 = 0;
    map_table<W>(a, S);
    __syncthreads();

    // this thread's bitmap words; nothing may be set at or past n_c
    bool bad = false;
    const uint32_t b0 = tid * BB;
    uint32_t bw[NW];
    if (layout == DCR_LAYOUT_LIST) {
        // the thread's elements [e_lo, e_lo + 8 BB): find the first listed
        // index at or past e_lo, then set the bits of the indices below the
        // end; the list must ascend strictly (checked pairwise across the
        // workgroup); bits past n_c are refused below
        const uint16_t* lst = reinterpret_cast<const uint16_t*>(S.stage);
        const uint32_t e_lo = b0 * 8, e_hi = e_lo + BB * 8;
        uint32_t l = 0, h = K;
        while (l < h) {
            const uint32_t m = (l + h) >> 1;
            if (lst[m] < e_lo) l = m + 1;
            else h = m;
        }
#pragma unroll
        for (uint32_t i = 0; i < NW; i++) bw[i] = 0;
        for (uint32_t j = l; j < K && lst[j] < e_hi; j++) {
            const uint32_t e = lst[j] - e_lo;
#pragma unroll
            for (uint32_t i = 0; i < NW; i++) bw[i] |= (e >> 5) == i ? (1u << (e & 31u)) : 0u;
        }
        for (uint32_t j = tid; j + 1 < K; j += kSmallThreads)
            if (lst[j] >= lst[j + 1]) bad = true;
    } else {
        bitmap_slice<NW>(S, 0, b0, bm, bw);
    }
    const uint32_t cnt = checked_slice<NW>(bw, b0, n_c, bad);
    // a fused pair's overwrite record (bitmap layout, staged at sz): its own
    // slice and checks
    uint32_t bw2[NW];
    bool bad2 = false;
#pragma unroll
    for (uint32_t i = 0; i < NW; i++) bw2[i] = 0;
    if (fused) bitmap_slice<NW>(S, sz, b0, bm, bw2);
    const uint32_t cnt2 = checked_slice<NW>(bw2, b0, n_c, bad2);
    // SPARSE: presence words (one per thread), their prefix counts and H
    const uint32_t n_pw = dpad16((K + 7) / 8) / 4;
    uint32_t pword = 0;
    if (hm == DCR_HI_SPARSE && tid < n_pw) {
        pword = reinterpret_cast<const uint32_t*>(S.stage + pres)[tid];
        const uint32_t pb = tid * 32;
        const uint32_t vmask = pb >= K ? 0u : (K - pb >= 32 ? 0xFFFFFFFFu : ((1u << (K - pb)) - 1u));
        if (pword & ~vmask) bad = true;
    }
    // both records' counts in one scan, as the two 32-bit halves (a chunk's
    // changes stay far below 2^32)
    uint64_t total;
    const uint64_t jj = small_excl_scan(uint64_t(cnt) | (uint64_t(cnt2) << 32), total, S.scan);
    const uint32_t j = uint32_t(jj), j2 = uint32_t(jj >> 32);
    if (hm == DCR_HI_SPARSE) {
        uint64_t ptot;
        const uint32_t pp = uint32_t(small_excl_scan(__popc(pword), ptot, S.scan));
        if (tid < n_pw) S.pres_pre[tid] = pp;
        if (tid == 0 && ptot != H) bad = true;
    }
    if (tid == 0 && uint32_t(total) != K) bad = true;
    if (tid == 0 && fused && uint32_t(total >> 32) != S.ent2[2]) bad2 = true;
    if (bad) atomicOr(&S.bad, 1u);
    if (bad2) atomicOr(&S.bad2, 1u);
    __syncthreads();
    // a malformed record is refused before any write of its own
    const bool ok = S.bad == 0, ok2 = fused && S.bad2 == 0;
    if (!ok && !ok2) return;

    uint8_t* dst = reinterpret_cast<uint8_t*>(S.dst);
    // a fused pair's overwrite record (the format keeps a chunk's two
    // records to disjoint 16-byte groups): its sections in the stage
    const uint32_t K2 = S.ent2[2], hm2 = (S.ent2[3] >> 8) & 0xFF;
    const uint32_t lo2 = sz + bm, pk2 = dpad16(K2);
    if (!ok) {
        // this record refused: the overwrite record alone
        apply_groups<W, NW>(a, S, dst, n_c, bw2, j2, lo2, lo2 + pk2, lo2 + pk2, pk2, hm2, false);
        __syncthreads();
        if (tid == 0) a.flags[r + 1] = 1;   // never a retry
        return;
    }
    const uint32_t pk = dpad16(K);
    const bool is_xor = kind == DCR_KIND_XOR;
    // Line mode for records dense enough that most lines hold a change:
    // touched 128-byte lines are read and written whole.  Only lines no
    // other writer touches are written whole: the record is the only one of
    // this call for its chunk, or the chunk's other record (next to it in the
    // directory; records of a chunk mark disjoint groups) has its bitmap
    // staged, and lines it marks take the group-by-group update instead.  A
    // record applied by another call or by the large-record kernel does not
    // run concurrently.  The chunk is canonical at a 128-byte aligned
    // address (lines past the chunk's elements are never written whole).
    // A list record's bitmap is rebuilt past the record in the stage (each
    // thread stores its checked slice whole, so a slice that straddles the
    // bitmap's end needs room for all of it), when it fits.
    // A fused pair's two records are both this workgroup's: every touched
    // line may be written whole, each group patched from its own record.
    const uint32_t bmo = layout == DCR_LAYOUT_LIST ? dpad16(sz) : 0u;
    const bool line_mode = !a.sharded && (S.solo == 1 || S.sib || fused) && bmo + bm + BB <= kSmallStage &&
                           uint64_t(K) * kLineDensity >= n_c && (reinterpret_cast<uintptr_t>(dst) & 127u) == 0;
    if (!line_mode && ok2) apply_groups<W, NW>(a, S, dst, n_c, bw2, j2, lo2, lo2 + pk2, lo2 + pk2, pk2, hm2, false);
    if (line_mode) {
        S.jpre[tid] = j;
        S.jpre2[tid] = j2;
        if (layout == DCR_LAYOUT_LIST && b0 < bm) {
#pragma unroll
            for (uint32_t i = 0; i < NW; i++) reinterpret_cast<uint32_t*>(S.stage + bmo + b0)[i] = bw[i];
        }
        // lines that may be written whole: inside the chunk's elements and
        // unmarked by the other record
        const uint32_t whole_lines = n_c / (8 * V), sib = S.sib;
        for (uint32_t L = tid; L < kLinesPerChunk; L += kSmallThreads)
            S.whole[L] = L < whole_lines && !(sib && S.other[L]);
        __syncthreads();
        apply_lines<W>(S, dst, n_c, lo, hi, pres, pk, hm, is_xor, bmo, ok2, sz, lo2, pk2, hm2);
    } else {
        apply_groups<W, NW>(a, S, dst, n_c, bw, j, lo, hi, pres, pk, hm, is_xor);
    }
    __syncthreads();
    if (tid == 0 && !a.retry) {   // visible with the writes at kernel completion
        a.flags[r] = 1;
        if (ok2) a.flags[r + 1] = 1;
    }
}

// Thread 0 of a small-record workgroup: the other records of this call for
// the record's chunk (t, c), whose entries are adjacent in the directory
// (the XOR record first).  solo 1: none.  solo 2: exactly one, a bitmap
// record of the other kind whose bitmap lies inside the payload, at
// sib_off (if that record is malformed it is refused and writes nothing).
// solo 0: anything else.  pv / nx: the first halves of the neighbouring
// entries, de: this record's entry.  Values only (no reference to LDS or
// to a private array), so that every access keeps its address space.
struct Neighbours {
    uint32_t solo;
    uint64_t sib_off;
};
__device__ __forceinline__ Neighbours chunk_neighbours(const uint4* de, uint64_t r, uint64_t first, uint64_t end,
                                                       uint64_t payload_bytes, uint32_t t, uint32_t c, uint32_t kind,
                                                       uint32_t n_c, bool has_prev, bool has_next, uint4 pv, uint4 nx) {
    Neighbours o{0u, 0};
    const bool sp = has_prev && pv.x == t && pv.y == c;
    const bool sn = has_next && nx.x == t && nx.y == c;
    if (!sp && !sn) {
        o.solo = 1u;
        return o;
    }
    if (sp && sn) return o;
    const uint32_t ow = sp ? pv.w : nx.w;
    const uint32_t xk = sp ? (ow & 0xFF) : kind, ok = sp ? kind : (ow & 0xFF);
    if (xk != DCR_KIND_XOR || ok != DCR_KIND_OW || (ow >> 24) != DCR_LAYOUT_BITMAP) return o;
    // the entry past the other record names another chunk
    if (sp ? r >= first + 2 : r + 2 < end) {
        const uint4 far = sp ? de[-4] : de[4];
        if (far.x == t && far.y == c) return o;
    }
    const uint4 o1 = sp ? de[-1] : de[3];
    const uint64_t off = uint64_t(o1.x) | (uint64_t(o1.y) << 32);
    const uint64_t bm = dpad16((n_c + 7) / 8);
    if ((off & 15u) != 0 || off > payload_bytes || bm > payload_bytes - off) return o;
    o.solo = 2u;
    o.sib_off = off;
    return o;
}

// Thread 0 of a small-record workgroup: whether its record belongs to a
// fused pair, a chunk's XOR record and, next in the directory, its overwrite
// record, both in bitmap layout, structurally valid, staged together within
// kSmallStage, with no other record of this call for the chunk, in a
// canonical-layout apply.  The XOR record's workgroup applies both (and
// owns both records' flags and counts); the overwrite record's workgroup
// does nothing.  Both reach the same answer from the same entries.  e: the
// record's entry (already checked); pv / nx: the first halves of the
// previous / next entries (when they exist).  Returns 1 for the XOR record
// of a fused pair, with its partner's entry in e2; 2 for the overwrite
// record; 0 otherwise.
__device__ __forceinline__ uint32_t pair_role(const ApplyArgs& a, const uint4* de, uint64_t r, const uint32_t (&e)[8],
                                              bool has_prev, bool has_next, uint4 pv, uint4 nx, uint32_t (&e2)[8]) {
    if (a.sharded || a.retry) return 0;
    const uint64_t end = a.first + gridDim.x;
    const uint32_t t = e[0], c = e[1];
    const bool is_xor = (e[3] & 0xFF) == DCR_KIND_XOR;
    uint32_t x[8], o[8];
    if (is_xor) {
        if (!has_next || nx.x != t || nx.y != c) return 0;
        if (has_prev && pv.x == t && pv.y == c) return 0;
        if (r + 2 < end) {
            const uint4 f = de[4];
            if (f.x == t && f.y == c) return 0;
        }
        const uint4 n1 = de[3];
        const uint32_t oo[8] = {nx.x, nx.y, nx.z, nx.w, n1.x, n1.y, n1.z, n1.w};
        for (int i = 0; i < 8; i++) x[i] = e[i], o[i] = oo[i];
    } else {
        if (!has_prev || pv.x != t || pv.y != c) return 0;
        if (has_next && nx.x == t && nx.y == c) return 0;
        if (r >= a.first + 2) {
            const uint4 f = de[-4];
            if (f.x == t && f.y == c) return 0;
        }
        const uint4 p1 = de[-1];
        const uint32_t xx[8] = {pv.x, pv.y, pv.z, pv.w, p1.x, p1.y, p1.z, p1.w};
        for (int i = 0; i < 8; i++) x[i] = xx[i], o[i] = e[i];
    }
    if ((x[3] & 0xFF) != DCR_KIND_XOR || (o[3] & 0xFF) != DCR_KIND_OW) return 0;
    if ((x[3] >> 24) != DCR_LAYOUT_BITMAP || (o[3] >> 24) != DCR_LAYOUT_BITMAP) return 0;
    uint32_t nx_c, no_c;
    if (!entry_ok(a, x, nx_c) || !entry_ok(a, o, no_c)) return 0;
    if (uint64_t(x[6]) + o[6] > kSmallStage) return 0;
    const uint32_t Kx = x[2], hmx = (x[3] >> 8) & 0xFF;
    if (hmx == DCR_HI_SPARSE && dpad16((Kx + 7) / 8) / 4 > kSmallThreads) return 0;
    for (int i = 0; i < 8; i++) e2[i] = o[i];
    return is_xor ? 1u : 2u;
}

// Seven workgroups per compute unit: a small record's time is mostly the
// latency of its dependent loads (entry, record, lines), so more resident
// workgroups pay for the few registers spilled to reach them.  PAIRS: fused
// pairs are looked for (an apply; a retry's stream holds overwrite records
// only, and its build of the kernel carries none of the pair code).
template <bool PAIRS>
__global__ __launch_bounds__(kSmallThreads) __attribute__((amdgpu_waves_per_eu(7, 8))) void apply_small_kernel(
    ApplyArgs a) {
    __shared__ SmallShared S;
    const uint64_t r = a.first + blockIdx.x;
    uint32_t n_c = 0;
    if (threadIdx.x == 0) {
        const uint4* de = reinterpret_cast<const uint4*>(a.dir + r * DCR_DIRENT_BYTES);
        const uint4 e0 = de[0], e1 = de[1];
        // the neighbouring entries' (tensor, chunk), loaded with the entry
        // (a chunk's records are adjacent in the directory)
        const bool has_prev = r > a.first, has_next = r + 1 < a.first + gridDim.x;
        const uint4 pv = has_prev ? de[-2] : make_uint4(0xFFFFFFFFu, 0xFFFFFFFFu, 0, 0);
        const uint4 nx = has_next ? de[2] : make_uint4(0xFFFFFFFFu, 0xFFFFFFFFu, 0, 0);
        // the dedup flag, and the canonical tensor's address (needed by the
        // writes), loaded with the entry and with the tensor's descriptor
        // rather than one after the other
        const uint8_t done = a.retry ? uint8_t(0) : a.flags[r];
        const uint8_t* cbase = (!a.sharded && e0.x < a.n_tensors) ? a.canon[e0.x] : nullptr;
        uint32_t e[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
        uint32_t e2[8];
        uint32_t st, fused = 0, pskip = 0;
        uint64_t rec = r;
        const bool valid = entry_ok(a, e, n_c);
        const uint32_t role = PAIRS && valid ? pair_role(a, de, r, e, has_prev, has_next, pv, nx, e2) : 0u;
        if (role == 1) {
            // the XOR record of a fused pair: both records' dedup flags decide
            // which of the two this workgroup applies
            const bool done2 = a.flags[r + 1] != 0;
            if (done && done2) {
                pskip = 1;
            } else if (done) {
                // only the overwrite record, alone
                pskip = 1;
                rec = r + 1;
                for (int i = 0; i < 8; i++) e[i] = e2[i];
            } else if (done2) {
                pskip = 1;
            } else {
                fused = 1;
                for (int i = 0; i < 8; i++) S.ent2[i] = e2[i];
            }
        }
        for (int i = 0; i < 8; i++) S.ent[i] = e[i];
        if (!valid) {
            st = 0;
        } else if (role == 2) {
            st = 4;
        } else if (done && rec == r) {
            st = 1;
        } else {
            const uint32_t K = e[2], hm = (e[3] >> 8) & 0xFF;
            const bool fits = e[6] <= kSmallStage && (hm != DCR_HI_SPARSE || dpad16((K + 7) / 8) / 4 <= kSmallThreads);
            st = fits ? 2 : 3;
            if (!fits) a.big_list[atomicAdd(a.big_count, 1u)] = uint32_t(rec - a.first);
            else map_chunk(a, S, e[0], e[1]);
            const Neighbours nb = chunk_neighbours(de, r, a.first, a.first + gridDim.x, a.payload_bytes, e[0], e[1],
                                                   e[3] & 0xFF, n_c, has_prev, has_next, pv, nx);
            S.solo = nb.solo;
            S.sib_off = nb.sib_off;
            // line mode beside the other record, when this one is dense
            // enough for line mode
            S.sib = nb.solo == 2 && !a.sharded && uint64_t(K) * kLineDensity >= n_c ? 1u : 0u;
            if (rec != r) S.solo = S.sib = 0;   // a pair's overwrite record alone: the group path
            if (fused) S.sib = 0;               // both of the pair's records are this workgroup's
            S.dst = cbase ? reinterpret_cast<uint64_t>(cbase) + uint64_t(e[1]) * kChunkBytes : 0;
        }
        S.state = st;
        S.n_c = n_c;
        S.fused = fused;
        S.pskip = pskip;
        S.rec = rec;
    }
    __syncthreads();
    const uint32_t st = S.state;
    n_c = S.n_c;
    if (st >= 3) return;   // deferred, or applied by its pair's XOR record
    const uint64_t rec = S.rec;
    if (threadIdx.x == 0 && (S.pskip || st == 1))
        atomicAdd(reinterpret_cast<unsigned long long*>(&a.result->n_skipped),
                  (unsigned long long)((st == 1 ? 1u : 0u) + S.pskip));
    if (st == 1) return;
    if (st == 2) {
        const uint32_t w = (S.ent[3] >> 16) & 0xFF;
        if (w == 2) apply_small_record<2, PAIRS>(a, S, rec, n_c);
        else if (w == 1) apply_small_record<1, PAIRS>(a, S, rec, n_c);
        else apply_small_record<4, PAIRS>(a, S, rec, n_c);
        if (threadIdx.x == 0 && PAIRS && S.fused && S.bad2) {
            atomicAdd(reinterpret_cast<unsigned long long*>(&a.result->n_invalid), 1ull);
            atomicMin(reinterpret_cast<unsigned long long*>(&a.result->first_invalid), (unsigned long long)(rec + 1));
        }
        if (!S.bad) return;
    }
    if (threadIdx.x == 0) {
        atomicAdd(reinterpret_cast<unsigned long long*>(&a.result->n_invalid), 1ull);
        atomicMin(reinterpret_cast<unsigned long long*>(&a.result->first_invalid), (unsigned long long)rec);
    }
}

__global__ void apply_init_kernel(dcr_apply_result* res, uint32_t* big_count) {
    if (threadIdx.x == 0) {
        uint4* r = reinterpret_cast<uint4*>(res);
        r[0] = make_uint4(0, 0, 0, 0);
        r[1] = make_uint4(0, 0, 0xFFFFFFFFu, 0xFFFFFFFFu);
        *big_count = 0;
    }
}

// Every record of the call ends applied, skipped or refused.
__global__ void apply_finalize_kernel(dcr_apply_result* res, uint64_t n) {
    if (threadIdx.x == 0) res->n_applied = n - res->n_skipped - res->n_invalid;
}

// ------------------------------------------------------------- host side

static int32_t fail(int32_t rc, const std::string& m) {
    set_error(m);
    return rc;
}
static bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// compute units of the current device
static uint32_t cu_count() {
    static uint32_t cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = uint32_t(n);
    }
    return cached[dev];
}

// Device memory of the allocation-free encode (dcr_encode_noalloc): its
// workspace and staging area.  In host code `scratch` names a host-side
// stand-in, not the device array: its device address, one per GPU, comes
// from hipGetSymbolAddress with that GPU current, and only that address is
// handed to kernels and copies.
static __device__ __align__(256) uint8_t scratch[DCR_NOALLOC_SCRATCH_BYTES];
static std::atomic<uint8_t*> g_scratch_ptr[64];
static std::mutex g_scratch_mu;

// The current device's copy of `scratch` (looked up once per device).
static int32_t scratch_ptr(uint8_t** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(DCR_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(DCR_E_INVAL, "device index out of range for the scratch table");
    uint8_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            void* q = nullptr;
            e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !q)
                return fail(DCR_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
            p = static_cast<uint8_t*>(q);
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return DCR_OK;
}

// benchmark hook: events recorded around the main kernel of each call
static thread_local hipEvent_t g_ev_start = nullptr, g_ev_stop = nullptr;
static void mark(bool start, hipStream_t s) {
    hipEvent_t e = start ? g_ev_start : g_ev_stop;
    if (g_ev_start && g_ev_stop) (void)hipEventRecord(e, s);
}
static int32_t hip_check(hipError_t e, const char* what) {
    if (e == hipSuccess) return DCR_OK;
    return fail(DCR_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

template <class T>
static const T* tab(const Plan& p, uint64_t off) {
    return reinterpret_cast<const T*>(static_cast<const uint8_t*>(p.dev_tables) + off);
}

static int32_t copy_ptrs(void* dst, const void* const* src, uint64_t n, hipStream_t s) {
    if (!n) return DCR_OK;
    return hip_check(hipMemcpyAsync(dst, src, n * sizeof(void*), hipMemcpyHostToDevice, s), "pointer table copy");
}

static int32_t check_header(const Plan& p, const dcr_stream_header* h, uint64_t expected_base) {
    if (!h) return fail(DCR_E_INVAL, "header is NULL");
    if (h->magic != DCR_MAGIC || h->format_version != DCR_FORMAT_VERSION || h->chunk_bytes != DCR_CHUNK_BYTES ||
        h->reserved0 != 0 || h->reserved1 != 0)
        return fail(DCR_E_FORMAT, "stream header: bad magic / version / chunk size");
    if (h->stream_kind > DCR_MODE_RETRY) return fail(DCR_E_FORMAT, "stream header: bad stream kind");
    if (h->plan_fingerprint != p.fingerprint) return fail(DCR_E_FORMAT, "stream header: plan fingerprint mismatch");
    if (h->base_version != expected_base) return fail(DCR_E_VERSION, "stream base_version != expected base version");
    return DCR_OK;
}

// canon: one pointer per canonical tensor, or with `sharded` one per shard
// of the plan (a receiver layout: records go through the plan's pieces).
static int32_t launch_apply(const dcr_plan* plan, void* const* canon, const dcr_stream_header* hdr,
                            const void* dir, const void* payload, uint8_t* flags, uint64_t first, uint64_t n,
                            dcr_apply_result* res, void* ws, uint64_t ws_bytes, hipStream_t s, bool retry,
                            bool sharded = false) {
    const Plan& p = *plan;
    const uint32_t nT = uint32_t(p.tensors.size());
    const uint32_t nS = uint32_t(p.shard_bytes.size());
    if ((n && !dir) || (n && !payload) || !res || !ws) return fail(DCR_E_INVAL, "NULL device buffer");
    if (!al16(dir) || !al16(payload) || !al16(res) || !al16(ws)) return fail(DCR_E_INVAL, "buffer not 16-byte aligned");
    if (!retry && n && !flags) return fail(DCR_E_INVAL, "applied_flags is NULL");
    if (ws_bytes < p.ws_bytes) return fail(DCR_E_CAPACITY, "workspace too small");
    // one workgroup per record in one grid (work-items must fit 32 bits): at
    // most kSmallThreads-wide workgroups for a call within the plan's record
    // capacity, kThreads-wide ones beyond it
    if (n > (n <= p.big_cap ? UINT32_MAX / kSmallThreads : UINT32_MAX / kThreads))
        return fail(DCR_E_INVAL, "too many records in one call");
    uint8_t* wsb = static_cast<uint8_t*>(ws);
    int32_t rc;
    if (sharded) {
        if (!p.shard_disjoint)
            return fail(DCR_E_INVAL, "receiver layout maps two canonical elements to one shard element");
        if (nS && !canon) return fail(DCR_E_INVAL, "shards is NULL");
        for (uint32_t i = 0; i < nS; i++) {
            if (p.shard_bytes[i] && !canon[i]) return fail(DCR_E_INVAL, "shard " + std::to_string(i) + " is NULL");
            if (!al16(canon[i])) return fail(DCR_E_INVAL, "shard " + std::to_string(i) + " not 16-byte aligned");
        }
        rc = copy_ptrs(wsb + p.ws_old, reinterpret_cast<const void* const*>(canon), nS, s);
    } else {
        if (nT && !canon) return fail(DCR_E_INVAL, "canon is NULL");
        for (uint32_t t = 0; t < nT; t++) {
            if (p.tensors[t].numel && !canon[t]) return fail(DCR_E_INVAL, "canonical tensor " + std::to_string(t) + " is NULL");
            if (!al16(canon[t])) return fail(DCR_E_INVAL, "canonical tensor " + std::to_string(t) + " not 16-byte aligned");
        }
        rc = copy_ptrs(wsb + p.ws_canon, reinterpret_cast<const void* const*>(canon), nT, s);
    }
    if (rc) return rc;
    uint32_t* big_count = reinterpret_cast<uint32_t*>(wsb + p.ws_counter) + kCtrBig;
    hipLaunchKernelGGL(apply_init_kernel, dim3(1), dim3(64), 0, s, res, big_count);
    if (n) {
        ApplyArgs a;
        a.tensors = tab<DevTensor>(p, p.off_tensors);
        a.canon = reinterpret_cast<uint8_t* const*>(wsb + p.ws_canon);
        a.dir = static_cast<const uint8_t*>(dir);
        a.payload = static_cast<const uint8_t*>(payload);
        a.flags = flags;
        a.result = res;
        a.big_list = reinterpret_cast<uint32_t*>(wsb + p.ws_big);
        a.big_count = big_count;
        a.payload_bytes = hdr->payload_bytes;
        a.first = first;
        a.n_tensors = nT;
        a.retry = retry ? 1u : 0u;
        a.sharded = sharded ? 1u : 0u;
        a.rchunks = tab<DevChunk>(p, p.off_chunks);
        a.rpieces = tab<DevPiece>(p, p.off_pieces);
        a.rshards = reinterpret_cast<uint8_t* const*>(wsb + p.ws_old);
        mark(true, s);
        if (n <= p.big_cap) {
            // small records with many per compute unit; the rest deferred
            if (a.retry) hipLaunchKernelGGL(apply_small_kernel<false>, dim3(uint32_t(n)), dim3(kSmallThreads), 0, s, a);
            else hipLaunchKernelGGL(apply_small_kernel<true>, dim3(uint32_t(n)), dim3(kSmallThreads), 0, s, a);
            hipLaunchKernelGGL(apply_big_kernel, dim3(uint32_t(std::min<uint64_t>(n, 2 * cu_count()))), dim3(kThreads),
                               0, s, a);
        } else {
            hipLaunchKernelGGL(apply_kernel, dim3(uint32_t(n)), dim3(kThreads), 0, s, a);
        }
        mark(false, s);
    }
    hipLaunchKernelGGL(apply_finalize_kernel, dim3(1), dim3(64), 0, s, res, n);
    return hip_check(hipGetLastError(), "apply launch");
}

}  // namespace dcr

extern "C" {

void dcr_set_kernel_events(void* start, void* stop) {
    dcr::g_ev_start = static_cast<hipEvent_t>(start);
    dcr::g_ev_stop = static_cast<hipEvent_t>(stop);
}

int32_t dcr_plan_upload(dcr_plan* plan, void* dev_tables, uint64_t bytes, void* stream) {
    using namespace dcr;
    set_error("");
    if (!plan || !dev_tables) return fail(DCR_E_INVAL, "NULL argument");
    if (!al16(dev_tables)) return fail(DCR_E_INVAL, "dev_tables not 16-byte aligned");
    if (bytes < plan->table_bytes) return fail(DCR_E_CAPACITY, "dev_tables too small");
    int32_t rc = hip_check(hipMemcpyAsync(dev_tables, plan->blob.data(), plan->table_bytes, hipMemcpyHostToDevice,
                                          static_cast<hipStream_t>(stream)),
                           "plan upload");
    if (rc) return rc;
    plan->dev_tables = dev_tables;
    return DCR_OK;
}

}  // extern "C"

namespace dcr {

// The encode.  delta_dir / delta_flags / n_delta: a partial retry (mode
// RETRY restricted to the chunks with an unflagged record of that DELTA
// directory); n_delta == UINT64_MAX for a whole encode.
static int32_t encode_impl(const dcr_plan* plan, const void* const* old_shards, const void* const* new_shards,
                           uint32_t mode, uint64_t base_version, uint64_t new_version, void* header_dev,
                           void* dir_dev, uint64_t dir_cap, void* payload_dev, uint64_t payload_cap,
                           dcr_encode_result* result_dev, void* workspace_dev, uint64_t ws_bytes, void* stream,
                           const uint8_t* delta_dir, const uint8_t* delta_flags, uint64_t n_delta,
                           uint32_t n_slices = 0, uint8_t* ready_dev = nullptr) {
    if (!plan) return fail(DCR_E_INVAL, "plan is NULL");
    const Plan& p = *plan;
    if (!p.dev_tables) return fail(DCR_E_INVAL, "plan not uploaded");
    const uint32_t lists = (mode & DCR_ENC_INDEX_LISTS) ? 1u : 0u;
    mode &= ~uint32_t(DCR_ENC_INDEX_LISTS);
    if (mode > DCR_MODE_RETRY) return fail(DCR_E_INVAL, "bad mode");
    if (!header_dev || !result_dev || !workspace_dev) return fail(DCR_E_INVAL, "NULL device buffer");
    if ((dir_cap && !dir_dev) || (payload_cap && !payload_dev)) return fail(DCR_E_INVAL, "NULL device buffer");
    if (!al16(header_dev) || !al16(dir_dev) || !al16(payload_dev) || !al16(result_dev) || !al16(workspace_dev))
        return fail(DCR_E_INVAL, "buffer not 16-byte aligned");
    if (ws_bytes < p.ws_bytes) return fail(DCR_E_CAPACITY, "workspace too small");
    const uint32_t nS = uint32_t(p.shard_bytes.size());
    if (nS && (!old_shards || !new_shards)) return fail(DCR_E_INVAL, "shard arrays are NULL");
    for (uint32_t s = 0; s < nS; s++) {
        if (p.shard_bytes[s] && (!old_shards[s] || !new_shards[s]))
            return fail(DCR_E_INVAL, "shard " + std::to_string(s) + " is NULL");
        if (!al16(old_shards[s]) || !al16(new_shards[s]))
            return fail(DCR_E_INVAL, "shard " + std::to_string(s) + " not 16-byte aligned");
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace_dev);
    int32_t rc = copy_ptrs(ws + p.ws_old, old_shards, nS, s);
    if (!rc) rc = copy_ptrs(ws + p.ws_new, new_shards, nS, s);
    if (rc) return rc;
    const uint32_t n_tiles = uint32_t(p.chunks.size());
    // look-back status words and counters start at zero
    const uint64_t n_zero = (p.ws_old) / 8;
    hipLaunchKernelGGL(fill_u64_kernel, dim3(uint32_t(std::min<uint64_t>((n_zero + 255) / 256, 4096))), dim3(256), 0,
                       s, reinterpret_cast<uint64_t*>(ws), n_zero, 0ull);
    const bool partial = n_delta != UINT64_MAX;
    uint64_t* need = reinterpret_cast<uint64_t*>(ws + p.ws_need);
    if (partial && n_delta)
        hipLaunchKernelGGL(retry_need_kernel, dim3(uint32_t(std::min<uint64_t>((n_delta + 255) / 256, 4096))),
                           dim3(256), 0, s, delta_dir, delta_flags, n_delta, tab<DevTensor>(p, p.off_tensors),
                           uint32_t(p.tensors.size()), need, reinterpret_cast<uint32_t*>(ws + p.ws_counter));
    const auto* tensors = tab<DevTensor>(p, p.off_tensors);
    const auto* chunks = tab<DevChunk>(p, p.off_chunks);
    const auto* pieces = tab<DevPiece>(p, p.off_pieces);
    const auto* old_sh = reinterpret_cast<const uint8_t* const*>(ws + p.ws_old);
    const auto* new_sh = reinterpret_cast<const uint8_t* const*>(ws + p.ws_new);
    auto* scale_flags = reinterpret_cast<uint64_t*>(ws + p.ws_scale);
    if (mode == DCR_MODE_DELTA && !p.scale_chunks.empty())
        hipLaunchKernelGGL(scale_flags_kernel, dim3(uint32_t(p.scale_chunks.size())), dim3(256), 0, s, tensors,
                           chunks, pieces, tab<uint32_t>(p, p.off_scale_chunks), old_sh, new_sh, scale_flags);
    uint32_t* counter = reinterpret_cast<uint32_t*>(ws + p.ws_counter);
    // bytes past the plan's workspace: staging area.  When it holds every
    // chunk's worst-case slot (max_payload_bytes), each tile writes to its
    // own fixed slot.  A smaller one of at least compact_stage_bytes is used
    // compactly: it is cut into kStageParts partitions, and each tile with
    // records claims exactly their bytes in its workgroup's partition with one
    // atomic add; a tile that finds no room writes nothing, and after the
    // fix-up (which knows every offset) it is encoded again straight to its
    // place.  Anything smaller (or a sliced encode without the whole area):
    // the in-order encode, no staging.
    uint8_t* stage = ws + p.ws_bytes;
    const uint64_t stage_bytes = ws_bytes - p.ws_bytes;
    const bool full = stage_bytes >= p.max_payload_bytes;
    const bool compact = !full && !n_slices && n_tiles && stage_bytes >= p.compact_stage_bytes;
    const uint32_t staged = (full || compact) ? 1u : 0u;
    EncodeArgs a;
    a.tensors = tensors;
    a.chunks = chunks;
    a.pieces = pieces;
    a.old_sh = old_sh;
    a.new_sh = new_sh;
    a.scale_flags = scale_flags;
    a.status = reinterpret_cast<uint64_t*>(ws + p.ws_status);
    a.counter = counter;
    a.tile_agg = reinterpret_cast<uint64_t*>(ws + p.ws_agg);
    a.tile_info = reinterpret_cast<uint64_t*>(ws + p.ws_info);
    a.slots = tab<uint64_t>(p, p.off_slots);
    a.stage = stage;
    a.dir = static_cast<uint8_t*>(dir_dev);
    a.payload = static_cast<uint8_t*>(payload_dev);
    a.dir_cap = dir_cap;
    a.payload_cap = payload_cap;
    a.need = partial ? need : nullptr;
    a.soff = reinterpret_cast<uint64_t*>(ws + p.ws_soff);
    a.stage_ctr = reinterpret_cast<unsigned long long*>(ws + p.ws_counter + kStageCtrOff);
    a.part_bytes = (stage_bytes / kStageParts) & ~uint64_t(15);
    a.n_tiles = n_tiles;
    a.mode = mode;
    a.lists = lists;
    a.compact = compact ? 1u : 0u;
    FixArgs f;
    f.tensors = tensors;
    f.chunks = chunks;
    f.tile_agg = a.tile_agg;
    f.tile_info = a.tile_info;
    f.slots = a.slots;
    f.need = a.need;
    f.soff = a.soff;
    f.redo = reinterpret_cast<uint32_t*>(ws + p.ws_status);   // the tile look-back status is unused when staged
    f.redo_count = reinterpret_cast<uint32_t*>(ws + p.ws_counter + kRedoCtrOff);
    f.fix_status = reinterpret_cast<uint64_t*>(ws + p.ws_fix);
    f.counter = counter;
    f.stage = stage;
    f.dir = a.dir;
    f.payload = a.payload;
    f.dir_cap = dir_cap;
    f.payload_cap = payload_cap;
    f.n_tiles = n_tiles;
    f.n_blocks = (n_tiles + kFixTiles - 1) / kFixTiles;
    f.staged = staged;
    f.lists = lists;
    f.compact = a.compact;
    // one direct tile kernel: width index i (1-, 2-, 4-byte), index lists,
    // compact staging
    auto launch_direct = [&](int i, bool li, bool co, uint32_t n, const uint32_t* list) {
#define DCR_DIRECT(W_, L_, C_) \
    hipLaunchKernelGGL((encode_direct_kernel<W_, L_, C_>), dim3(n), dim3(kThreads), 0, s, a, list, n)
        const int key = i * 4 + (li ? 2 : 0) + (co ? 1 : 0);
        switch (key) {
            case 0: DCR_DIRECT(1, false, false); break;
            case 1: DCR_DIRECT(1, false, true); break;
            case 2: DCR_DIRECT(1, true, false); break;
            case 3: DCR_DIRECT(1, true, true); break;
            case 4: DCR_DIRECT(2, false, false); break;
            case 5: DCR_DIRECT(2, false, true); break;
            case 6: DCR_DIRECT(2, true, false); break;
            case 7: DCR_DIRECT(2, true, true); break;
            case 8: DCR_DIRECT(4, false, false); break;
            case 9: DCR_DIRECT(4, false, true); break;
            case 10: DCR_DIRECT(4, true, false); break;
            default: DCR_DIRECT(4, true, true); break;
        }
#undef DCR_DIRECT
    };
    // Tiles [t0, t1): in a staged launch the direct tiles of each element
    // width, then the others (any order: every tile has its own slot); the
    // lists hold tile ids in ascending order, so a range of tiles is a range
    // of each list.  In order: one workgroup per tile, tile ids taken from a
    // counter that carries over from the previous range.
    auto run_tiles = [&](uint32_t t0, uint32_t t1, bool timed) {
        if (timed) mark(true, s);
        if (staged) {
            for (int i = 0; i < 3; i++) {
                const auto& L = p.direct[i];
                const uint32_t lo = uint32_t(std::lower_bound(L.begin(), L.end(), t0) - L.begin());
                const uint32_t n = uint32_t(std::lower_bound(L.begin(), L.end(), t1) - L.begin()) - lo;
                if (!n) continue;
                const uint32_t* list = tab<uint32_t>(p, p.off_direct[i]) + lo;
                launch_direct(i, lists != 0, compact, n, list);
            }
        } else if (t1 > t0) {
            const dim3 g(t1 - t0), b(kThreads);
            switch (p.widths) {
                case 1: hipLaunchKernelGGL(encode_kernel<1>, g, b, 0, s, a); break;
                case 2: hipLaunchKernelGGL(encode_kernel<2>, g, b, 0, s, a); break;
                case 3: hipLaunchKernelGGL(encode_kernel<3>, g, b, 0, s, a); break;
                case 4: hipLaunchKernelGGL(encode_kernel<4>, g, b, 0, s, a); break;
                case 5: hipLaunchKernelGGL(encode_kernel<5>, g, b, 0, s, a); break;
                case 6: hipLaunchKernelGGL(encode_kernel<6>, g, b, 0, s, a); break;
                default: hipLaunchKernelGGL(encode_kernel<7>, g, b, 0, s, a); break;
            }
        }
        if (timed) mark(false, s);
        if (staged) {
            const auto& L = p.slow;
            const uint32_t lo = uint32_t(std::lower_bound(L.begin(), L.end(), t0) - L.begin());
            const uint32_t n = uint32_t(std::lower_bound(L.begin(), L.end(), t1) - L.begin()) - lo;
            if (n)
                hipLaunchKernelGGL(encode_slow_kernel, dim3(n), dim3(kThreads), 0, s, a,
                                   tab<uint32_t>(p, p.off_slow) + lo, n);
        }
    };
    // fix-up blocks [b0, b1); block ids come from a counter that carries over
    auto run_fix = [&](uint32_t b0, uint32_t b1) {
        if (b1 > b0) hipLaunchKernelGGL(encode_fixup_kernel, dim3(b1 - b0), dim3(kFixTiles), 0, s, f);
    };
    auto finalize = [&]() {
        hipLaunchKernelGGL(encode_finalize_kernel, dim3(1), dim3(64), 0, s, counter, mode, base_version, new_version,
                           p.fingerprint, dir_cap, payload_cap, static_cast<uint8_t*>(header_dev), result_dev);
    };
    if (!n_slices) {
        if (n_tiles) {
            run_tiles(0, n_tiles, true);
            run_fix(0, f.n_blocks);
            if (compact) {
                const dim3 g(std::min<uint32_t>(n_tiles, 2 * cu_count()));
                hipLaunchKernelGGL(encode_redo_kernel<2>, g, dim3(kThreads), 0, s, a, f.redo, f.redo_count);
                hipLaunchKernelGGL(encode_redo_kernel<1>, g, dim3(kThreads), 0, s, a, f.redo, f.redo_count);
                hipLaunchKernelGGL(encode_redo_kernel<4>, g, dim3(kThreads), 0, s, a, f.redo, f.redo_count);
            }
        }
        finalize();
    } else {
        // slice k: fix-up blocks [k * nb / n_slices, (k + 1) * nb / n_slices)
        // and their tiles; the last slice also finalises the header before it
        // is published
        const uint32_t nb = f.n_blocks;
        for (uint32_t k = 0; k < n_slices; k++) {
            const uint32_t b0 = uint32_t(uint64_t(k) * nb / n_slices), b1 = uint32_t(uint64_t(k + 1) * nb / n_slices);
            const uint32_t t0 = b0 * kFixTiles, t1 = std::min(b1 * kFixTiles, n_tiles);
            run_tiles(t0, t1, false);
            run_fix(b0, b1);
            if (k + 1 == n_slices) finalize();
            hipLaunchKernelGGL(publish_kernel, dim3(1), dim3(64), 0, s, f.fix_status, b1 > b0 ? b1 - 1 : UINT32_MAX,
                               counter, mode, base_version, new_version, p.fingerprint, dir_cap, payload_cap, ready_dev,
                               k);
        }
    }
    return hip_check(hipGetLastError(), "encode launch");
}

}  // namespace dcr

extern "C" {

int32_t dcr_encode(const dcr_plan* plan, const void* const* old_shards, const void* const* new_shards, uint32_t mode,
                   uint64_t base_version, uint64_t new_version, void* header_dev, void* dir_dev, uint64_t dir_cap,
                   void* payload_dev, uint64_t payload_cap, dcr_encode_result* result_dev, void* workspace_dev,
                   uint64_t ws_bytes, void* stream) {
    using namespace dcr;
    set_error("");
    return encode_impl(plan, old_shards, new_shards, mode, base_version, new_version, header_dev, dir_dev, dir_cap,
                       payload_dev, payload_cap, result_dev, workspace_dev, ws_bytes, stream, nullptr, nullptr,
                       UINT64_MAX);
}

int32_t dcr_encode_noalloc(const dcr_plan* plan, const void* const* old_shards, const void* const* new_shards,
                           uint32_t mode, uint64_t base_version, uint64_t new_version, void* header_dev,
                           void* dir_dev, uint64_t dir_cap, void* payload_dev, uint64_t payload_cap,
                           dcr_encode_result* result_dev, void* stream) {
    using namespace dcr;
    set_error("");
    if (!plan) return fail(DCR_E_INVAL, "plan is NULL");
    if (plan->ws_bytes > DCR_NOALLOC_SCRATCH_BYTES)
        return fail(DCR_E_CAPACITY, "plan workspace of " + std::to_string(plan->ws_bytes) +
                                        " bytes exceeds the library's scratch of " +
                                        std::to_string(uint64_t(DCR_NOALLOC_SCRATCH_BYTES)) + " bytes");
    uint8_t* ws = nullptr;
    const int32_t rc = scratch_ptr(&ws);
    if (rc) return rc;
    // staged when every chunk's slot fits past the workspace, else in order
    // (a compact area of what is left could be far below a large stream's
    // size, and would then encode most chunks twice)
    const uint64_t ws_bytes = plan->ws_bytes + plan->max_payload_bytes <= DCR_NOALLOC_SCRATCH_BYTES
                                  ? uint64_t(DCR_NOALLOC_SCRATCH_BYTES)
                                  : plan->ws_bytes;
    return encode_impl(plan, old_shards, new_shards, mode, base_version, new_version, header_dev, dir_dev, dir_cap,
                       payload_dev, payload_cap, result_dev, ws, ws_bytes, stream, nullptr, nullptr, UINT64_MAX);
}

int32_t dcr_encode_pipelined(const dcr_plan* plan, const void* const* old_shards, const void* const* new_shards,
                             uint32_t mode, uint64_t base_version, uint64_t new_version, void* header_dev,
                             void* dir_dev, uint64_t dir_cap, void* payload_dev, uint64_t payload_cap,
                             dcr_encode_result* result_dev, void* workspace_dev, uint64_t ws_bytes,
                             uint32_t n_slices, void* ready_host, uint64_t ready_bytes, void* stream) {
    using namespace dcr;
    set_error("");
    if (!plan) return fail(DCR_E_INVAL, "plan is NULL");
    if (n_slices == 0) return fail(DCR_E_INVAL, "n_slices must be at least 1");
    if (!ready_host || (reinterpret_cast<uintptr_t>(ready_host) & 63u))
        return fail(DCR_E_INVAL, "ready region is NULL or not 64-byte aligned");
    const uint32_t nb = uint32_t((plan->chunks.size() + kFixTiles - 1) / kFixTiles);
    const uint32_t n_eff = std::min(n_slices, std::max(nb, 1u));
    if (ready_bytes < 64 + 64 * uint64_t(n_eff)) return fail(DCR_E_CAPACITY, "ready region too small");
    // the kernels write the region through its device address; anything but
    // pinned host memory is refused before any launch
    hipPointerAttribute_t at{};
    if (hipPointerGetAttributes(&at, ready_host) != hipSuccess || at.type != hipMemoryTypeHost || !at.devicePointer) {
        (void)hipGetLastError();
        return fail(DCR_E_INVAL, "ready region is not pinned host memory (hipHostMalloc)");
    }
    auto* r = static_cast<uint8_t*>(ready_host);
    __atomic_store_n(reinterpret_cast<int32_t*>(r + 8), 0, __ATOMIC_RELAXED);
    __atomic_store_n(reinterpret_cast<uint32_t*>(r + 12), n_eff, __ATOMIC_RELAXED);
    __atomic_store_n(reinterpret_cast<uint64_t*>(r), uint64_t(0), __ATOMIC_RELEASE);
    return encode_impl(plan, old_shards, new_shards, mode, base_version, new_version, header_dev, dir_dev, dir_cap,
                       payload_dev, payload_cap, result_dev, workspace_dev, ws_bytes, stream, nullptr, nullptr,
                       UINT64_MAX, n_eff, static_cast<uint8_t*>(at.devicePointer));
}

int32_t dcr_ready_wait(const void* ready_host, uint32_t slice, uint64_t timeout_us, dcr_stream_header* out) {
    using namespace dcr;
    set_error("");
    if (!ready_host || !out) return fail(DCR_E_INVAL, "NULL argument");
    const auto* r = static_cast<const uint8_t*>(ready_host);
    const uint32_t n = __atomic_load_n(reinterpret_cast<const uint32_t*>(r + 12), __ATOMIC_RELAXED);
    if (slice >= n) return fail(DCR_E_INVAL, "slice " + std::to_string(slice) + " of " + std::to_string(n));
    const auto t0 = std::chrono::steady_clock::now();
    for (uint64_t spin = 0;; spin++) {
        if (__atomic_load_n(reinterpret_cast<const uint64_t*>(r), __ATOMIC_ACQUIRE) > slice) {
            std::memcpy(out, r + 64 + 64 * uint64_t(slice), sizeof(dcr_stream_header));
            return DCR_OK;
        }
        const int32_t st = __atomic_load_n(reinterpret_cast<const int32_t*>(r + 8), __ATOMIC_ACQUIRE);
        if (st) return fail(st, "the encode stopped publishing (status " + std::to_string(st) + ")");
        if ((spin & 255u) == 255u) {
            const uint64_t us = uint64_t(std::chrono::duration_cast<std::chrono::microseconds>(
                                              std::chrono::steady_clock::now() - t0).count());
            if (us >= timeout_us) return fail(DCR_E_TIMEOUT, "slice " + std::to_string(slice) + " not published");
            std::this_thread::sleep_for(std::chrono::microseconds(5));
        }
    }
}

int32_t dcr_encode_retry_partial(const dcr_plan* plan, const void* const* old_shards, const void* const* new_shards,
                                 const dcr_stream_header* delta_header, const void* delta_dir_dev,
                                 uint64_t delta_dir_bytes, const uint8_t* delta_flags_dev, uint64_t base_version,
                                 uint64_t new_version, void* header_dev, void* dir_dev, uint64_t dir_cap,
                                 void* payload_dev, uint64_t payload_cap, dcr_encode_result* result_dev,
                                 void* workspace_dev, uint64_t ws_bytes, void* stream) {
    using namespace dcr;
    set_error("");
    if (!plan) return fail(DCR_E_INVAL, "plan is NULL");
    if (!delta_header) return fail(DCR_E_INVAL, "delta header is NULL");
    int32_t rc = check_header(*plan, delta_header, delta_header->base_version);
    if (rc) return rc;
    if (delta_header->stream_kind != DCR_MODE_DELTA) return fail(DCR_E_FORMAT, "not a DELTA stream");
    const uint64_t n = delta_header->n_records;
    if (n > delta_dir_bytes / DCR_DIRENT_BYTES) return fail(DCR_E_INVAL, "delta directory smaller than n_records");
    if (n && (!delta_dir_dev || !delta_flags_dev)) return fail(DCR_E_INVAL, "NULL delta directory or flags");
    if (!al16(delta_dir_dev)) return fail(DCR_E_INVAL, "delta directory not 16-byte aligned");
    return encode_impl(plan, old_shards, new_shards, DCR_MODE_RETRY, base_version, new_version, header_dev, dir_dev,
                       dir_cap, payload_dev, payload_cap, result_dev, workspace_dev, ws_bytes, stream,
                       static_cast<const uint8_t*>(delta_dir_dev), delta_flags_dev, n);
}

int32_t dcr_apply(const dcr_plan* plan, void* const* canon, const dcr_stream_header* header, const void* dir_dev,
                  const void* payload_dev, uint8_t* applied_flags_dev, uint64_t first_record, uint64_t n_records,
                  uint64_t expected_base_version, dcr_apply_result* result_dev, void* workspace_dev,
                  uint64_t ws_bytes, void* stream) {
    using namespace dcr;
    set_error("");
    if (!plan) return fail(DCR_E_INVAL, "plan is NULL");
    if (!plan->dev_tables) return fail(DCR_E_INVAL, "plan not uploaded");
    int32_t rc = check_header(*plan, header, expected_base_version);
    if (rc) return rc;
    if (first_record > header->n_records || n_records > header->n_records - first_record)
        return fail(DCR_E_INVAL, "record range outside the stream");
    return launch_apply(plan, canon, header, dir_dev, payload_dev, applied_flags_dev, first_record, n_records,
                        result_dev, workspace_dev, ws_bytes, static_cast<hipStream_t>(stream), false);
}

int32_t dcr_apply_overwrite_retry(const dcr_plan* plan, void* const* canon, const dcr_stream_header* header,
                                  const void* dir_dev, const void* payload_dev, uint64_t expected_base_version,
                                  dcr_apply_result* result_dev, void* workspace_dev, uint64_t ws_bytes,
                                  void* stream) {
    using namespace dcr;
    set_error("");
    if (!plan) return fail(DCR_E_INVAL, "plan is NULL");
    if (!plan->dev_tables) return fail(DCR_E_INVAL, "plan not uploaded");
    int32_t rc = check_header(*plan, header, expected_base_version);
    if (rc) return rc;
    if (header->stream_kind != DCR_MODE_RETRY) return fail(DCR_E_FORMAT, "not a RETRY stream");
    return launch_apply(plan, canon, header, dir_dev, payload_dev, nullptr, 0, header->n_records, result_dev,
                        workspace_dev, ws_bytes, static_cast<hipStream_t>(stream), true);
}

int32_t dcr_apply_sharded(const dcr_plan* plan, void* const* shards, const dcr_stream_header* header,
                          const void* dir_dev, const void* payload_dev, uint8_t* applied_flags_dev,
                          uint64_t first_record, uint64_t n_records, uint64_t expected_base_version,
                          dcr_apply_result* result_dev, void* workspace_dev, uint64_t ws_bytes, void* stream) {
    using namespace dcr;
    set_error("");
    if (!plan) return fail(DCR_E_INVAL, "plan is NULL");
    if (!plan->dev_tables) return fail(DCR_E_INVAL, "plan not uploaded");
    int32_t rc = check_header(*plan, header, expected_base_version);
    if (rc) return rc;
    if (first_record > header->n_records || n_records > header->n_records - first_record)
        return fail(DCR_E_INVAL, "record range outside the stream");
    return launch_apply(plan, shards, header, dir_dev, payload_dev, applied_flags_dev, first_record, n_records,
                        result_dev, workspace_dev, ws_bytes, static_cast<hipStream_t>(stream), false, true);
}

int32_t dcr_apply_overwrite_retry_sharded(const dcr_plan* plan, void* const* shards,
                                          const dcr_stream_header* header, const void* dir_dev,
                                          const void* payload_dev, uint64_t expected_base_version,
                                          dcr_apply_result* result_dev, void* workspace_dev, uint64_t ws_bytes,
                                          void* stream) {
    using namespace dcr;
    set_error("");
    if (!plan) return fail(DCR_E_INVAL, "plan is NULL");
    if (!plan->dev_tables) return fail(DCR_E_INVAL, "plan not uploaded");
    int32_t rc = check_header(*plan, header, expected_base_version);
    if (rc) return rc;
    if (header->stream_kind != DCR_MODE_RETRY) return fail(DCR_E_FORMAT, "not a RETRY stream");
    return launch_apply(plan, shards, header, dir_dev, payload_dev, nullptr, 0, header->n_records, result_dev,
                        workspace_dev, ws_bytes, static_cast<hipStream_t>(stream), true, true);
}

}  // extern "C"
