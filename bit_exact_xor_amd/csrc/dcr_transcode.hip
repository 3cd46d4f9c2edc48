// dcr_transcode.hip -- a RETRY stream written from a DELTA stream and the old
// shards, without reading the new shards.
//
// After a failed refit the whole change set is sent again as overwrites
// (tokendh blog, "no backup copy"; ai.info abstract): per
// changed chunk, one overwrite record with the new bits of every changed
// element.  The DELTA stream of the same step already names every changed
// element of a chunk, with either its XOR mask (new = old ^ mask) or its new
// bits, so the chunk's RETRY record is its DELTA records merged in element
// order, with old folded into the XOR changes.  Old is read at the changed
// elements only.  The result is the stream a RETRY encode from old and new
// writes, byte for byte.
//
// Launch sequence (one stream): zero the per-chunk tables and counters;
// index the DELTA directory (validate, find each chunk's first record, size
// its RETRY record); scan the sizes in plan order (block sums, one-workgroup
// scan of the sums, block rescans); write each record (one 256-thread
// workgroup per chunk); write the header and the result.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>

#include "dcr_internal.h"

namespace dcr {
namespace {

constexpr uint32_t kTT = 256;                          // threads of the record kernel
constexpr uint32_t kCached = 64;                       // pieces of a chunk resolved in LDS
constexpr uint32_t kScanT = 1024, kScanPer = 4, kScanBlock = kScanT * kScanPer;
constexpr uint32_t kValBits = 36;                      // scan value: records << 36 | bytes / 16
constexpr uint64_t kValMask = (uint64_t(1) << kValBits) - 1;
// 64-bit counters in the workspace's counter area
constexpr uint32_t kTotal = 0, kTotalK = 1, kErr = 2, kNCtr = 32;
constexpr unsigned long long kErrFormat = 1;

__device__ __forceinline__ uint32_t p16(uint32_t x) { return (x + 15u) & ~15u; }

// Bytes of a DELTA record given its directory fields; 0 when the fields do
// not describe a record of the format.
__device__ uint32_t delta_record_bytes(uint32_t w, uint32_t n_c, uint32_t K, uint32_t kind, uint32_t hm,
                                       uint32_t H, uint32_t layout) {
    if (K == 0 || K > n_c || kind > DCR_KIND_OW || layout > DCR_LAYOUT_LIST) return 0;
    const uint32_t sz = (layout == DCR_LAYOUT_LIST ? p16(2 * K) : p16((n_c + 7) / 8)) + p16(K);
    if (w == 1) return (hm == DCR_HI_NONE && H == 0) ? sz : 0;
    if (kind == DCR_KIND_OW) return (hm == DCR_HI_DENSE && H == K) ? sz + (w - 1) * p16(K) : 0;
    if (w != 2) return 0;   // XOR records hold 1- or 2-byte elements
    if (hm == DCR_HI_NONE) return H == 0 ? sz : 0;
    if (hm == DCR_HI_DENSE) return H == K ? sz + p16(K) : 0;
    if (hm == DCR_HI_SPARSE) return (H >= 1 && H <= K) ? sz + p16((K + 7) / 8) + p16(H) : 0;
    return 0;
}

// First section of an overwrite record with K changes: the index list when
// the encode option asks for lists and it is strictly smaller, else the bitmap.
__device__ __forceinline__ uint32_t retry_sec0(uint32_t n_c, uint32_t K, uint32_t lists) {
    const uint32_t bm = p16((n_c + 7) / 8);
    return (lists && p16(2 * K) < bm) ? p16(2 * K) : bm;
}

__device__ __forceinline__ uint32_t chunk_elems(const DevTensor& td, uint32_t c) {
    const uint64_t E = kChunkBytes / td.w;
    const uint64_t rem = td.numel - uint64_t(c) * E;
    return uint32_t(rem < E ? rem : E);
}

__global__ __launch_bounds__(256) void tx_fill_kernel(uint64_t* p, uint64_t n) {
    for (uint64_t i = uint64_t(blockIdx.x) * 256u + threadIdx.x; i < n; i += uint64_t(gridDim.x) * 256u) p[i] = 0;
}

// One thread per DELTA record: check the entry, its order and its size; for
// the first record of each chunk store first[tile] = index + 1 | Ktot << 32
// and val[tile] = 1 << 36 | (RETRY record bytes) / 16.
__global__ __launch_bounds__(256) void tx_index_kernel(const uint8_t* dir, uint64_t n, uint64_t payload_bytes,
                                                       const DevTensor* tensors, uint32_t n_tensors, uint32_t lists,
                                                       uint64_t* first, uint64_t* val, unsigned long long* ctr) {
    const uint64_t i = uint64_t(blockIdx.x) * 256u + threadIdx.x;
    if (i >= n) return;
    const uint4* de = reinterpret_cast<const uint4*>(dir + i * DCR_DIRENT_BYTES);
    const uint4 a = de[0], b = de[1];
    bool ok = a.x < n_tensors;
    DevTensor td{};
    uint32_t n_c = 0;
    if (ok) {
        td = tensors[a.x];
        ok = a.y < td.n_chunks;
    }
    if (ok) {
        n_c = chunk_elems(td, a.y);
        const uint32_t kind = a.w & 0xFF, hm = (a.w >> 8) & 0xFF, eb = (a.w >> 16) & 0xFF, layout = a.w >> 24;
        const uint64_t off = uint64_t(b.x) | (uint64_t(b.y) << 32);
        const uint32_t sz = delta_record_bytes(td.w, n_c, a.z, kind, hm, b.w, layout);
        ok = eb == td.w && sz != 0 && sz == b.z && (off & 15u) == 0 && off <= payload_bytes &&
             sz <= payload_bytes - off;
    }
    // records ascend by (tensor, chunk); a chunk holds an XOR record and
    // then an overwrite record at most
    bool is_first = true;
    uint64_t Ktot = a.z;
    if (ok && i > 0) {
        const uint4 p = de[-2];
        if (p.x == a.x && p.y == a.y) {
            is_first = false;
            ok = (p.w & 0xFF) == DCR_KIND_XOR && (a.w & 0xFF) == DCR_KIND_OW;
        } else {
            ok = p.x < a.x || (p.x == a.x && p.y < a.y);
        }
    }
    if (ok && i + 1 < n) {
        const uint4 q = de[2];
        if (q.x == a.x && q.y == a.y) {
            if (!is_first) ok = false;   // a third record of the chunk
            else Ktot += q.z;
        }
    }
    if (ok && Ktot > n_c) ok = false;
    if (!ok) {
        atomicOr(ctr + kErr, kErrFormat);
        return;
    }
    if (is_first) {
        const uint32_t tile = td.first_chunk + a.y;
        const uint32_t K = uint32_t(Ktot);
        first[tile] = (i + 1) | (Ktot << 32);
        const uint32_t sz = retry_sec0(n_c, K, lists) + td.w * p16(K);
        val[tile] = (uint64_t(1) << kValBits) | (sz >> 4);
    }
}

// Sum of 1024 values in LDS (all threads; ends with every thread holding it).
__device__ uint64_t scan_block_sum(uint64_t v, uint64_t* s) {
    const uint32_t tid = threadIdx.x;
    s[tid] = v;
    __syncthreads();
    for (uint32_t h = kScanT / 2; h > 0; h >>= 1) {
        if (tid < h) s[tid] += s[tid + h];
        __syncthreads();
    }
    const uint64_t r = s[0];
    __syncthreads();
    return r;
}

// Exclusive prefix of v over the 1024 threads (Hillis-Steele in LDS).
__device__ uint64_t scan_block_excl(uint64_t v, uint64_t* s, uint64_t& total) {
    const uint32_t tid = threadIdx.x;
    s[tid] = v;
    __syncthreads();
    for (uint32_t d = 1; d < kScanT; d <<= 1) {
        const uint64_t y = tid >= d ? s[tid - d] : 0;
        __syncthreads();
        s[tid] += y;
        __syncthreads();
    }
    total = s[kScanT - 1];
    const uint64_t r = s[tid] - v;
    __syncthreads();
    return r;
}

// Block sums: bsum[2 b] = sum of val, bsum[2 b + 1] = sum of Ktot over the
// block's kScanBlock tiles.
__global__ __launch_bounds__(kScanT) void tx_reduce_kernel(const uint64_t* val, const uint64_t* first, uint64_t n,
                                                           uint64_t* bsum) {
    __shared__ uint64_t s[kScanT];
    const uint64_t t0 = uint64_t(blockIdx.x) * kScanBlock + uint64_t(threadIdx.x) * kScanPer;
    uint64_t v = 0, k = 0;
    for (uint32_t j = 0; j < kScanPer; j++) {
        if (t0 + j < n) {
            v += val[t0 + j];
            k += first[t0 + j] >> 32;
        }
    }
    v = scan_block_sum(v, s);
    k = scan_block_sum(k, s);
    if (threadIdx.x == 0) {
        bsum[2 * blockIdx.x] = v;
        bsum[2 * blockIdx.x + 1] = k;
    }
}

// One workgroup: exclusive scan of the block sums in place; totals to the
// counters.
__global__ __launch_bounds__(kScanT) void tx_scan_sums_kernel(uint64_t* bsum, uint64_t nb, unsigned long long* ctr) {
    __shared__ uint64_t s[kScanT];
    uint64_t carry = 0, ksum = 0;
    for (uint64_t base = 0; base < nb; base += kScanT) {
        const uint64_t b = base + threadIdx.x;
        const uint64_t v = b < nb ? bsum[2 * b] : 0;
        const uint64_t k = b < nb ? bsum[2 * b + 1] : 0;
        uint64_t tot = 0;
        const uint64_t ex = scan_block_excl(v, s, tot);
        ksum += scan_block_sum(k, s);
        if (b < nb) bsum[2 * b] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0) {
        ctr[kTotal] = carry;
        ctr[kTotalK] = ksum;
    }
}

// Rescan each block with its prefix: val[tile] becomes the tile's exclusive
// prefix (records << 36 | bytes / 16).  When the stream fits and the
// directory is well formed, each chunk with a record also gets a descriptor
// for the record kernel, written into the output directory slot its entry
// will take (32 bytes: DELTA record index, tile, prefix (2 words), first
// piece, piece count, elements | width << 24, 0).
__global__ __launch_bounds__(kScanT) void tx_downsweep_kernel(uint64_t* val, uint64_t n, const uint64_t* bsum,
                                                              const uint64_t* first, const DevChunk* chunks,
                                                              const DevTensor* tensors,
                                                              const unsigned long long* ctr, uint8_t* out_dir,
                                                              uint64_t dir_cap, uint64_t payload_cap) {
    __shared__ uint64_t s[kScanT];
    const uint64_t t0 = uint64_t(blockIdx.x) * kScanBlock + uint64_t(threadIdx.x) * kScanPer;
    uint64_t v[kScanPer], sum = 0;
    for (uint32_t j = 0; j < kScanPer; j++) {
        v[j] = t0 + j < n ? val[t0 + j] : 0;
        sum += v[j];
    }
    uint64_t tot = 0;
    uint64_t run = bsum[2 * blockIdx.x] + scan_block_excl(sum, s, tot);
    const uint64_t all = ctr[kTotal];
    const bool desc = !ctr[kErr] && (all >> kValBits) * DCR_DIRENT_BYTES <= dir_cap &&
                      ((all & kValMask) << 4) <= payload_cap;
    for (uint32_t j = 0; j < kScanPer; j++) {
        const uint64_t tile = t0 + j;
        if (tile < n) {
            val[tile] = run;
            if (desc && v[j]) {
                const DevChunk ch = chunks[tile];
                const DevTensor td = tensors[ch.tensor];
                const uint32_t n_c = chunk_elems(td, ch.chunk_idx);
                uint4* de = reinterpret_cast<uint4*>(out_dir + (run >> kValBits) * DCR_DIRENT_BYTES);
                de[0] = uint4{uint32_t(first[tile]) - 1u, uint32_t(tile), uint32_t(run), uint32_t(run >> 32)};
                de[1] = uint4{ch.first_piece, ch.n_pieces & kPiecesMask, n_c | (td.w << 24), 0u};
            }
        }
        run += v[j];
    }
}

__device__ __forceinline__ uint32_t shfl_up32(uint32_t v, uint32_t d) { return __shfl_up(v, d, 64); }

// Exclusive prefix of v over the kTT threads of the record kernel; total in
// `total`.  Contains two barriers.
__device__ uint64_t rec_scan(uint64_t v, uint64_t* red, uint64_t& total) {
    const uint32_t lane = threadIdx.x & 63u, wv = threadIdx.x >> 6;
    uint64_t x = v;
    for (uint32_t d = 1; d < 64; d <<= 1) {
        const uint64_t y = uint64_t(shfl_up32(uint32_t(x), d)) | (uint64_t(shfl_up32(uint32_t(x >> 32), d)) << 32);
        if (lane >= d) x += y;
    }
    if (lane == 63) red[wv] = x;
    __syncthreads();
    uint64_t base = 0, tot = 0;
    for (uint32_t k = 0; k < kTT / 64; k++) {
        const uint64_t r = red[k];
        if (k < wv) base += r;
        tot += r;
    }
    total = tot;
    __syncthreads();
    return base + x - v;
}

struct TxArgs {
    const uint8_t* dir;          // DELTA directory
    const uint8_t* payload;      // DELTA payload
    uint64_t n;                  // DELTA records
    const DevPiece* pieces;
    const uint8_t* const* old_sh;
    unsigned long long* ctr;
    uint8_t* out_dir;
    uint8_t* out_payload;
    uint64_t dir_cap, payload_cap;
    uint32_t lists;
    uint32_t maxw;               // bitmap words of the plan's largest chunk
};

// LDS of the record kernel, sized at launch for the plan's largest chunk
// bitmap (maxw words) and, with 2-byte tensors, the largest presence bitmap
// (presw words): this fixed part, then M (changed elements of the chunk, both
// records), B (those of the overwrite record when the chunk has two) and pre
// (per word: exclusive count of M | of B << 16), maxw words each, then pp
// (per presence word of the XOR record: exclusive count).
struct TxShared {
    uint64_t paddr[kCached];          // resolved pieces: shard address of canonical element canon_start
    uint64_t red[kTT / 64];
    uint32_t pstart[kCached];
};
constexpr uint32_t kTxFixed = (sizeof(uint64_t) * (kCached + kTT / 64) + sizeof(uint32_t) * kCached + 15) & ~15u;

// Address of chunk element e in the old shards.
__device__ __forceinline__ const uint8_t* old_elem(const TxArgs& a, const TxShared& S, uint32_t fp, uint32_t np,
                                                   uint32_t w, uint32_t e) {
    uint32_t l = 0, h = np;
    if (np <= kCached) {
        while (h - l > 1) {
            const uint32_t m = (l + h) >> 1;
            if (S.pstart[m] <= e) l = m;
            else h = m;
        }
        return reinterpret_cast<const uint8_t*>(S.paddr[l]) + uint64_t(e - S.pstart[l]) * w;
    }
    const DevPiece* pc = a.pieces + fp;
    while (h - l > 1) {
        const uint32_t m = (l + h) >> 1;
        if (pc[m].canon_start <= e) l = m;
        else h = m;
    }
    const DevPiece p = pc[l];
    return a.old_sh[p.shard] + (p.shard_elem_off + (e - p.canon_start)) * w;
}

// One workgroup per DELTA record; the first record of each chunk writes the
// chunk's RETRY record and directory entry.
__global__ __launch_bounds__(kTT) __attribute__((amdgpu_waves_per_eu(8, 8))) void tx_record_kernel(TxArgs a) {
    extern __shared__ __align__(16) uint8_t tx_lds[];
    TxShared& S = *reinterpret_cast<TxShared*>(tx_lds);
    uint32_t* const M = reinterpret_cast<uint32_t*>(tx_lds + kTxFixed);
    uint32_t* const B = M + a.maxw;
    uint32_t* const pre = B + a.maxw;
    uint32_t* const pp = pre + a.maxw;
    const uint32_t tid = threadIdx.x;
    // the counters and this record's descriptor in one round of loads (the
    // descriptor is valid when r is below the record count and the stream fits)
    const uint64_t r = blockIdx.x;
    if ((r + 1) * DCR_DIRENT_BYTES > a.dir_cap) return;
    const uint64_t err = a.ctr[kErr], tot = a.ctr[kTotal];
    const uint32_t* ds = reinterpret_cast<const uint32_t*>(a.out_dir + r * DCR_DIRENT_BYTES);
    const uint32_t ds0 = ds[0], ds2 = ds[2], ds3 = ds[3], fp = ds[4], np = ds[5], ds6 = ds[6];
    if (err || r >= (tot >> kValBits) || (tot >> kValBits) * DCR_DIRENT_BYTES > a.dir_cap ||
        ((tot & kValMask) << 4) > a.payload_cap)
        return;
    const uint64_t i = ds0;
    const uint64_t eo = uint64_t(ds2) | (uint64_t(ds3) << 32);
    const uint32_t n_c = ds6 & 0xFFFFFFu, w = ds6 >> 24;
    const uint32_t* d = reinterpret_cast<const uint32_t*>(a.dir + i * DCR_DIRENT_BYTES);
    const uint32_t t = d[0], c = d[1];
    const uint32_t nw = (n_c + 31) / 32;            // bitmap words holding elements
    const uint32_t bmb = p16((n_c + 7) / 8);        // bitmap section bytes
    const uint32_t nwp = bmb / 4;
    const bool two = i + 1 < a.n && d[8] == t && d[9] == c;
    // record A (the first), record B (the overwrite record after an XOR one)
    const uint32_t KA = d[2], kindA = d[3] & 0xFF, hmA = (d[3] >> 8) & 0xFF, layA = d[3] >> 24;
    const uint64_t offA = uint64_t(d[4]) | (uint64_t(d[5]) << 32);
    const uint32_t HA = d[7];
    const uint32_t KB = two ? d[10] : 0u, layB = two ? (d[11] >> 24) : 0u;
    const uint32_t Ktot = KA + KB;
    const uint64_t offB = two ? (uint64_t(d[12]) | (uint64_t(d[13]) << 32)) : 0u;
    const uint32_t s0A = layA == DCR_LAYOUT_LIST ? p16(2 * KA) : bmb, pkA = p16(KA);
    const uint32_t s0B = layB == DCR_LAYOUT_LIST ? p16(2 * KB) : bmb, pkB = p16(KB);
    const bool sparse = w == 2 && kindA == DCR_KIND_XOR && hmA == DCR_HI_SPARSE;
    const uint32_t presA = s0A + pkA;               // presence bits of A (SPARSE)
    const uint32_t npw = sparse ? (KA + 31) / 32 : 0u;
    const uint8_t* PA = a.payload + offA;
    const uint8_t* PB = a.payload + offB;

    // the change sets: bitmap records word by word (the padding words past
    // the chunk's elements too: a bit there is refused, as apply refuses it),
    // then index lists
    bool bad = false;
    for (uint32_t wi = tid; wi < nwp; wi += kTT) {
        uint32_t xa = 0, xb = 0;
        const uint32_t valid =
            wi >= nw ? 0u : (n_c - 32 * wi >= 32 ? 0xFFFFFFFFu : ((1u << (n_c - 32 * wi)) - 1u));
        if (layA == DCR_LAYOUT_BITMAP) xa = reinterpret_cast<const uint32_t*>(PA)[wi];
        if (two && layB == DCR_LAYOUT_BITMAP) xb = reinterpret_cast<const uint32_t*>(PB)[wi];
        if (((xa | xb) & ~valid) || (xa & xb)) bad = true;
        M[wi] = (xa | xb) & valid;
        B[wi] = xb & valid;
    }
    // the chunk's pieces (read only for XOR changes, after the bitmaps)
    if (np <= kCached && tid < np) {
        const DevPiece p = a.pieces[fp + tid];
        S.pstart[tid] = p.canon_start;
        S.paddr[tid] = reinterpret_cast<uint64_t>(a.old_sh[p.shard]) + p.shard_elem_off * w;
    }
    __syncthreads();
    if (layA == DCR_LAYOUT_LIST || (two && layB == DCR_LAYOUT_LIST)) {
        for (uint32_t q = 0; q < 2; q++) {
            const bool isB = q == 1;
            if (isB ? !(two && layB == DCR_LAYOUT_LIST) : layA != DCR_LAYOUT_LIST) continue;
            const uint16_t* L = reinterpret_cast<const uint16_t*>(isB ? PB : PA);
            const uint32_t K = isB ? KB : KA;
            for (uint32_t k = tid; k < K; k += kTT) {
                const uint32_t e = L[k];
                if (e >= n_c || (k && L[k - 1] >= e)) {
                    bad = true;
                    continue;
                }
                atomicOr(&M[e >> 5], 1u << (e & 31));
                if (isB) atomicOr(&B[e >> 5], 1u << (e & 31));
            }
        }
        __syncthreads();
    }

    // counts per thread: its words of M and B and its presence words of A
    const uint32_t wpt = (nw + kTT - 1) / kTT, w0 = tid * wpt, w1 = min(nw, w0 + wpt);
    const uint32_t ppt = (npw + kTT - 1) / kTT, q0 = tid * ppt, q1 = min(npw, q0 + ppt);
    uint32_t cM = 0, cB = 0, cP = 0;
    for (uint32_t wi = w0; wi < w1; wi++) {
        cM += __popc(M[wi]);
        cB += __popc(B[wi]);
    }
    for (uint32_t pw = q0; pw < q1; pw++) {
        uint32_t x = reinterpret_cast<const uint32_t*>(PA + presA)[pw];
        const uint32_t vm = KA - 32 * pw >= 32 ? 0xFFFFFFFFu : ((1u << (KA - 32 * pw)) - 1u);
        if (x & ~vm) bad = true;
        cP += __popc(x & vm);
    }
    uint64_t total = 0;
    const uint64_t ex = rec_scan(uint64_t(cM) | (uint64_t(cB) << 21) | (uint64_t(cP) << 42), S.red, total);
    {
        uint32_t rM = uint32_t(ex & 0x1FFFFF), rB = uint32_t((ex >> 21) & 0x1FFFFF), rP = uint32_t(ex >> 42);
        for (uint32_t wi = w0; wi < w1; wi++) {
            pre[wi] = rM | (rB << 16);
            rM += __popc(M[wi]);
            rB += __popc(B[wi]);
        }
        for (uint32_t pw = q0; pw < q1; pw++) {
            pp[pw] = rP;
            const uint32_t vm = KA - 32 * pw >= 32 ? 0xFFFFFFFFu : ((1u << (KA - 32 * pw)) - 1u);
            rP += __popc(reinterpret_cast<const uint32_t*>(PA + presA)[pw] & vm);
        }
    }
    const uint32_t tM = uint32_t(total & 0x1FFFFF), tB = uint32_t((total >> 21) & 0x1FFFFF);
    const uint32_t tP = uint32_t(total >> 42);
    if (tM != Ktot || tB != KB || tM != KA + KB || (sparse && tP != HA)) bad = true;
    if (__syncthreads_or(bad ? 1 : 0)) {   // also the barrier before the tables are read
        if (tid == 0) atomicOr(a.ctr + kErr, kErrFormat);
        return;
    }

    // the RETRY record
    const uint64_t rec = eo >> kValBits;
    uint8_t* out = a.out_payload + ((eo & kValMask) << 4);
    const uint32_t s0o = retry_sec0(n_c, Ktot, a.lists), pko = p16(Ktot);
    const bool listo = s0o != bmb;
    for (uint32_t wi = w0; wi < w1; wi++) {
        uint32_t m = M[wi];
        const uint32_t bb = B[wi];
        uint32_t r = pre[wi] & 0xFFFFu, rb = pre[wi] >> 16;
        while (m) {
            const uint32_t bit = uint32_t(__ffs(m) - 1);
            m &= m - 1;
            const uint32_t e = 32 * wi + bit;
            const bool isB = (bb >> bit) & 1u;
            const uint32_t j = isB ? rb : r - rb;
            const uint8_t* P = isB ? PB : PA;
            const uint32_t s0 = isB ? s0B : s0A, pk = isB ? pkB : pkA;
            const bool xr = !isB && kindA == DCR_KIND_XOR;
            uint32_t v = P[s0 + j];
            if (w == 2) {
                if (!xr || hmA == DCR_HI_DENSE) {
                    v |= uint32_t(P[s0 + pk + j]) << 8;
                } else if (hmA == DCR_HI_SPARSE) {
                    const uint32_t pwd = reinterpret_cast<const uint32_t*>(P + presA)[j >> 5];
                    if ((pwd >> (j & 31)) & 1u) {
                        const uint32_t rank = pp[j >> 5] + __popc(pwd & ((1u << (j & 31)) - 1u));
                        v |= uint32_t(P[presA + p16((KA + 7) / 8) + rank]) << 8;
                    }
                }
            } else if (w == 4) {
                v |= (uint32_t(P[s0 + pk + j]) << 8) | (uint32_t(P[s0 + 2 * pk + j]) << 16) |
                     (uint32_t(P[s0 + 3 * pk + j]) << 24);
            }
            if (xr) {
                const uint8_t* op = old_elem(a, S, fp, np, w, e);
                const uint32_t o = w == 1 ? uint32_t(*op)
                                          : (w == 2 ? uint32_t(*reinterpret_cast<const uint16_t*>(op))
                                                    : *reinterpret_cast<const uint32_t*>(op));
                v ^= o;
            }
            if (listo) reinterpret_cast<uint16_t*>(out)[r] = uint16_t(e);
            for (uint32_t pb = 0; pb < w; pb++) out[s0o + pb * pko + r] = uint8_t(v >> (8 * pb));
            r++;
            if (isB) rb++;
        }
    }
    // first section and zero padding
    if (!listo) {
        for (uint32_t wi = tid; wi < nwp; wi += kTT) reinterpret_cast<uint32_t*>(out)[wi] = M[wi];
    } else {
        for (uint32_t k = Ktot + tid; k < s0o / 2; k += kTT) reinterpret_cast<uint16_t*>(out)[k] = 0;
    }
    const uint32_t padn = pko - Ktot;
    for (uint32_t k = tid; k < padn * w; k += kTT) out[s0o + (k / padn) * pko + Ktot + k % padn] = 0;
    if (tid == 0) {
        const uint64_t off = (eo & kValMask) << 4;
        const uint32_t hm = w == 1 ? DCR_HI_NONE : DCR_HI_DENSE;
        uint4* de = reinterpret_cast<uint4*>(a.out_dir + rec * DCR_DIRENT_BYTES);
        de[0] = uint4{t, c, Ktot, DCR_KIND_OW | (hm << 8) | (w << 16) | ((listo ? DCR_LAYOUT_LIST : 0u) << 24)};
        de[1] = uint4{uint32_t(off), uint32_t(off >> 32), s0o + w * pko, w == 1 ? 0u : Ktot};
    }
}

__global__ void tx_finish_kernel(const unsigned long long* ctr, uint64_t base_version, uint64_t new_version,
                                 uint64_t fingerprint, uint64_t dir_cap, uint64_t payload_cap,
                                 dcr_stream_header* hdr, dcr_encode_result* res) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    const uint64_t tot = ctr[kTotal];
    const uint64_t n_rec = tot >> kValBits, bytes = (tot & kValMask) << 4;
    dcr_stream_header h{};
    h.magic = DCR_MAGIC;
    h.format_version = DCR_FORMAT_VERSION;
    h.stream_kind = DCR_MODE_RETRY;
    h.chunk_bytes = DCR_CHUNK_BYTES;
    h.base_version = base_version;
    h.new_version = new_version;
    h.plan_fingerprint = fingerprint;
    h.n_records = n_rec;
    h.payload_bytes = bytes;
    *hdr = h;
    dcr_encode_result r{};
    r.n_records = n_rec;
    r.payload_bytes = bytes;
    r.n_changed = ctr[kTotalK];
    r.status = ctr[kErr] ? DCR_E_FORMAT
                         : ((n_rec * DCR_DIRENT_BYTES > dir_cap || bytes > payload_cap) ? DCR_E_CAPACITY : DCR_OK);
    *res = r;
}

int32_t fail(int32_t rc, const std::string& m) {
    set_error(m);
    return rc;
}
bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace dcr

using namespace dcr;

extern "C" int32_t dcr_encode_retry_from_delta(
    const dcr_plan* plan, const void* const* old_shards, const dcr_stream_header* delta_header,
    const void* delta_dir_dev, uint64_t delta_dir_bytes, const void* delta_payload_dev,
    uint64_t delta_payload_bytes, uint32_t options, void* header_dev, void* dir_dev, uint64_t dir_cap,
    void* payload_dev, uint64_t payload_cap, dcr_encode_result* result_dev, void* workspace_dev,
    uint64_t ws_bytes, void* stream) {
    if (!plan) return fail(DCR_E_INVAL, "plan is NULL");
    const Plan& p = *plan;
    if (!p.dev_tables) return fail(DCR_E_INVAL, "plan not uploaded");
    if (options & ~uint32_t(DCR_ENC_INDEX_LISTS)) return fail(DCR_E_INVAL, "bad options");
    const dcr_stream_header* h = delta_header;
    if (!h) return fail(DCR_E_INVAL, "DELTA header is NULL");
    if (h->magic != DCR_MAGIC || h->format_version != DCR_FORMAT_VERSION || h->chunk_bytes != DCR_CHUNK_BYTES ||
        h->reserved0 != 0 || h->reserved1 != 0 || h->stream_kind != DCR_MODE_DELTA)
        return fail(DCR_E_FORMAT, "DELTA header: bad magic / version / chunk size / stream kind");
    if (h->plan_fingerprint != p.fingerprint) return fail(DCR_E_FORMAT, "DELTA header: plan fingerprint mismatch");
    const uint64_t n = h->n_records;
    // a valid DELTA stream holds at most an XOR and an overwrite record per
    // chunk (this also keeps the record kernel's grid within its limits)
    if (n > 2 * uint64_t(p.chunks.size()))
        return fail(DCR_E_FORMAT, "DELTA header: more records than two per chunk of the plan");
    if (n && (!delta_dir_dev || delta_dir_bytes / DCR_DIRENT_BYTES < n))
        return fail(DCR_E_INVAL, "DELTA directory buffer smaller than n_records entries");
    if (h->payload_bytes && (!delta_payload_dev || delta_payload_bytes < h->payload_bytes))
        return fail(DCR_E_INVAL, "DELTA payload buffer smaller than payload_bytes");
    if (!header_dev || !result_dev || !workspace_dev) return fail(DCR_E_INVAL, "NULL device buffer");
    if ((dir_cap && !dir_dev) || (payload_cap && !payload_dev)) return fail(DCR_E_INVAL, "NULL device buffer");
    if (!al16(header_dev) || !al16(dir_dev) || !al16(payload_dev) || !al16(result_dev) || !al16(workspace_dev) ||
        !al16(delta_dir_dev) || !al16(delta_payload_dev))
        return fail(DCR_E_INVAL, "buffer not 16-byte aligned");
    if (ws_bytes < p.ws_bytes) return fail(DCR_E_CAPACITY, "workspace too small");
    const uint32_t nS = uint32_t(p.shard_bytes.size());
    if (nS && !old_shards) return fail(DCR_E_INVAL, "shard array is NULL");
    for (uint32_t s = 0; s < nS; s++) {
        if (p.shard_bytes[s] && !old_shards[s]) return fail(DCR_E_INVAL, "shard " + std::to_string(s) + " is NULL");
        if (!al16(old_shards[s])) return fail(DCR_E_INVAL, "shard " + std::to_string(s) + " not 16-byte aligned");
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace_dev);
    if (nS) {
        const hipError_t e = hipMemcpyAsync(ws + p.ws_old, old_shards, nS * sizeof(void*), hipMemcpyHostToDevice, st);
        if (e != hipSuccess) return fail(DCR_E_HIP, std::string("pointer table copy: ") + hipGetErrorString(e));
    }
    const uint64_t n_tiles = p.chunks.size();
    const auto* tables = static_cast<const uint8_t*>(p.dev_tables);
    auto* first = reinterpret_cast<uint64_t*>(ws + p.ws_status);   // n_tiles entries
    auto* val = reinterpret_cast<uint64_t*>(ws + p.ws_agg);        // n_tiles entries
    auto* bsum = reinterpret_cast<uint64_t*>(ws + p.ws_fix);       // 2 per scan block
    auto* ctr = reinterpret_cast<unsigned long long*>(ws + p.ws_counter);
    const uint64_t nb = (n_tiles + kScanBlock - 1) / kScanBlock;
    hipLaunchKernelGGL(tx_fill_kernel, dim3(1), dim3(256), 0, st, reinterpret_cast<uint64_t*>(ctr), uint64_t(kNCtr));
    if (n_tiles) {
        const uint32_t g = uint32_t(std::min<uint64_t>((n_tiles + 255) / 256, 4096));
        hipLaunchKernelGGL(tx_fill_kernel, dim3(g), dim3(256), 0, st, first, n_tiles);
        hipLaunchKernelGGL(tx_fill_kernel, dim3(g), dim3(256), 0, st, val, n_tiles);
    }
    const auto* tensors = reinterpret_cast<const DevTensor*>(tables + p.off_tensors);
    const uint32_t lists = (options & DCR_ENC_INDEX_LISTS) ? 1u : 0u;
    if (n)
        hipLaunchKernelGGL(tx_index_kernel, dim3(uint32_t((n + 255) / 256)), dim3(256), 0, st,
                           static_cast<const uint8_t*>(delta_dir_dev), n, h->payload_bytes, tensors,
                           uint32_t(p.tensors.size()), lists, first, val, ctr);
    if (nb) hipLaunchKernelGGL(tx_reduce_kernel, dim3(uint32_t(nb)), dim3(kScanT), 0, st, val, first, n_tiles, bsum);
    hipLaunchKernelGGL(tx_scan_sums_kernel, dim3(1), dim3(kScanT), 0, st, bsum, nb, ctr);
    const auto* chunks = reinterpret_cast<const DevChunk*>(tables + p.off_chunks);
    if (nb)
        hipLaunchKernelGGL(tx_downsweep_kernel, dim3(uint32_t(nb)), dim3(kScanT), 0, st, val, n_tiles, bsum, first,
                           chunks, tensors, ctr, static_cast<uint8_t*>(dir_dev), dir_cap, payload_cap);
    if (n) {
        TxArgs a;
        a.dir = static_cast<const uint8_t*>(delta_dir_dev);
        a.payload = static_cast<const uint8_t*>(delta_payload_dev);
        a.n = n;
        a.pieces = reinterpret_cast<const DevPiece*>(tables + p.off_pieces);
        a.old_sh = reinterpret_cast<const uint8_t* const*>(ws + p.ws_old);
        a.ctr = ctr;
        a.out_dir = static_cast<uint8_t*>(dir_dev);
        a.out_payload = static_cast<uint8_t*>(payload_dev);
        a.dir_cap = dir_cap;
        a.payload_cap = payload_cap;
        a.lists = lists;
        // LDS for the largest chunk bitmap and (2-byte tensors) presence bitmap
        uint32_t maxw = 1, presw = 1;
        for (const DevTensor& td : p.dt) {
            const uint64_t E = kChunkBytes / td.w;
            const uint64_t ne = td.numel < E ? td.numel : E;
            maxw = std::max<uint32_t>(maxw, uint32_t((ne + 31) / 32));
            if (td.w == 2) presw = std::max<uint32_t>(presw, uint32_t((ne + 31) / 32));
        }
        a.maxw = (maxw + 3) & ~3u;
        const size_t lds = kTxFixed + sizeof(uint32_t) * (3 * size_t(a.maxw) + presw);
        hipLaunchKernelGGL(tx_record_kernel, dim3(uint32_t(n)), dim3(kTT), lds, st, a);
    }
    hipLaunchKernelGGL(tx_finish_kernel, dim3(1), dim3(64), 0, st, ctr, h->base_version, h->new_version,
                       p.fingerprint, dir_cap, payload_cap, static_cast<dcr_stream_header*>(header_dev), result_dev);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(DCR_E_HIP, std::string("launch: ") + hipGetErrorString(e));
    return DCR_OK;
}
