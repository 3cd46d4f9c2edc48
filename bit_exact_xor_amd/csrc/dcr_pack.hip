// dcr_pack.hip -- transport packing of a stream and its inverse.
//
// The pages compress the sparse mask stream before it travels (ai-feeds
// summary "key modules" 3; humansand "weight teleportation" page, "A strong
// baseline with Blackwell-native DE", on codecs for masks that are mostly
// runs of zeros).  Packing re-codes the first section of every index-list
// record as gap varints when that is strictly smaller, padded: the gap of
// change j is its index minus the previous change's index minus one (the
// first gap is the first index), written as unsigned LEB128 (seven bits per
// byte, low group first, the high bit set on every byte but the last), the
// varints back to back and zero-padded to 16 bytes; the directory entry gets
// layout DCR_LAYOUT_GAPS.  Every other section and record is copied as it is.
// Unpacking turns such records back into index lists; both write the header
// with the other magic and the new payload size.
//
// Launch sequence (one stream), the same for both directions: clear the
// counters; size every record (packing: a workgroup per record reads its
// list; unpacking: a thread per record, sizes follow from the entry); scan
// the sizes into output offsets (block sums, one workgroup over the sums,
// block rescans); write every record (a workgroup per record); write the
// header and the result.  The output directory holds per-record scratch
// (size, offset, section bytes, flags) until each record's own kernel
// replaces its slot with the final entry.
#include <hip/hip_runtime.h>

#include <string>

#include "dcr_internal.h"

namespace dcr {
namespace {

constexpr uint32_t kPT = 256;                    // threads of the per-record kernels
constexpr uint32_t kST = 1024;                   // threads of the scan kernels, one record each
constexpr uint32_t kMagicPacked = 0x50524344u;   // "DCRP"
// 64-bit counters at the workspace's counter area
constexpr uint32_t kPkTotal = 0, kPkErr = 1, kPkN = 4;
constexpr unsigned long long kErrFormat = 1;
// scratch flags
constexpr uint32_t kFValid = 1, kFGaps = 2;

__device__ __forceinline__ uint32_t p16(uint32_t x) { return (x + 15u) & ~15u; }
__device__ __forceinline__ uint32_t leb_len(uint32_t v) { return v < 0x80u ? 1u : (v < 0x4000u ? 2u : 3u); }

// Bytes of a record of layout 0 (bitmap) or 1 (index list) given its
// directory fields; 0 when the fields describe no record of the format.
__device__ uint32_t record_bytes(uint32_t w, uint32_t n_c, uint32_t K, uint32_t kind, uint32_t hm, uint32_t H,
                                 uint32_t layout) {
    if (K == 0 || K > n_c || kind > DCR_KIND_OW || layout > DCR_LAYOUT_LIST) return 0;
    const uint32_t sz = (layout == DCR_LAYOUT_LIST ? p16(2 * K) : p16((n_c + 7) / 8)) + p16(K);
    if (w == 1) return (hm == DCR_HI_NONE && H == 0) ? sz : 0;
    if (kind == DCR_KIND_OW) return (hm == DCR_HI_DENSE && H == K) ? sz + (w - 1) * p16(K) : 0;
    if (w != 2) return 0;
    if (hm == DCR_HI_NONE) return H == 0 ? sz : 0;
    if (hm == DCR_HI_DENSE) return H == K ? sz + p16(K) : 0;
    if (hm == DCR_HI_SPARSE) return (H >= 1 && H <= K && p16((K + 7) / 8) + p16(H) < p16(K)) ? sz + p16((K + 7) / 8) + p16(H) : 0;
    return 0;
}

// The entry's chunk: elements, or 0 when tensor / width / chunk do not exist.
__device__ uint32_t entry_n_c(const DevTensor* tensors, uint32_t n_tensors, uint32_t t, uint32_t c, uint32_t w) {
    if (t >= n_tensors) return 0;
    const DevTensor td = tensors[t];
    if (td.w != w || c >= td.n_chunks) return 0;
    const uint64_t E = kChunkBytes / w;
    const uint64_t rem = td.numel - uint64_t(c) * E;
    return uint32_t(rem < E ? rem : E);
}

struct Ent {
    uint32_t t, c, K, kind, hm, w, layout, sz, H;
    uint64_t off;
};

__device__ __forceinline__ Ent load_ent(const uint8_t* dir, uint64_t r) {
    const uint4* p = reinterpret_cast<const uint4*>(dir + r * DCR_DIRENT_BYTES);
    const uint4 a = p[0], b = p[1];
    Ent e;
    e.t = a.x;
    e.c = a.y;
    e.K = a.z;
    e.kind = a.w & 0xFFu;
    e.hm = (a.w >> 8) & 0xFFu;
    e.w = (a.w >> 16) & 0xFFu;
    e.layout = a.w >> 24;
    e.off = uint64_t(b.x) | (uint64_t(b.y) << 32);
    e.sz = b.z;
    e.H = b.w;
    return e;
}

__device__ __forceinline__ void store_ent(uint8_t* dir, uint64_t r, const Ent& e) {
    uint4* p = reinterpret_cast<uint4*>(dir + r * DCR_DIRENT_BYTES);
    p[0] = make_uint4(e.t, e.c, e.K, e.kind | (e.hm << 8) | (e.w << 16) | (e.layout << 24));
    p[1] = make_uint4(uint32_t(e.off), uint32_t(e.off >> 32), e.sz, e.H);
}

// scratch slot of record r in the output directory: u64 size, u64 offset
// (written by the scan), u32 section bytes, u32 flags
__device__ __forceinline__ void store_scratch(uint8_t* dir, uint64_t r, uint64_t size, uint32_t sec, uint32_t flags) {
    uint4* p = reinterpret_cast<uint4*>(dir + r * DCR_DIRENT_BYTES);
    p[0] = make_uint4(uint32_t(size), uint32_t(size >> 32), 0u, 0u);
    p[1] = make_uint4(sec, flags, 0u, 0u);
}

// Exclusive scan of one 32-bit value per thread of a kPT workgroup; sh holds
// kPT / 64 words.  Returns the prefix; total gets the sum.
__device__ uint32_t block_scan32(uint32_t v, uint32_t& total, uint32_t* sh) {
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    uint32_t x = v;
#pragma unroll
    for (uint32_t d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) sh[wave] = x;
    __syncthreads();
    uint32_t pre = 0, tot = 0;
#pragma unroll
    for (uint32_t w = 0; w < kPT / 64; w++) {
        pre += w < wave ? sh[w] : 0u;
        tot += sh[w];
    }
    __syncthreads();
    total = tot;
    return pre + x - v;
}

__global__ void pk_clear_kernel(unsigned long long* ctr) {
    if (threadIdx.x < kPkN) ctr[threadIdx.x] = 0;
}

// ---------------------------------------------------------------- sizes

// Packing: one workgroup per record.  Checks the entry (fields, size,
// bounds); for an index-list record, reads the list (indices below the
// chunk's elements, strictly ascending) and sums its gap varints' bytes.
__global__ __launch_bounds__(kPT) void pk_size_kernel(const DevTensor* tensors, uint32_t n_tensors, const uint8_t* dir,
                                                      const uint8_t* payload, uint64_t payload_bytes, uint8_t* out_dir,
                                                      unsigned long long* ctr) {
    __shared__ uint32_t sh[kPT / 64];
    __shared__ uint32_t s_ok, s_nc, s_bad;
    const uint64_t r = blockIdx.x;
    const uint32_t tid = threadIdx.x;
    const Ent e = load_ent(dir, r);   // uniform: every thread loads the entry
    if (tid == 0) {
        const uint32_t n_c = entry_n_c(tensors, n_tensors, e.t, e.c, e.w);
        const uint32_t want = n_c ? record_bytes(e.w, n_c, e.K, e.kind, e.hm, e.H, e.layout) : 0u;
        s_ok = (want != 0 && want == e.sz && (e.off & 15u) == 0 && e.off <= payload_bytes &&
                e.sz <= payload_bytes - e.off) ? 1u : 0u;
        s_nc = n_c;
        s_bad = 0;
    }
    __syncthreads();
    if (!s_ok) {
        if (tid == 0) {
            atomicOr(ctr + kPkErr, kErrFormat);
            store_scratch(out_dir, r, 0, 0, 0);
        }
        return;
    }
    if (e.layout != DCR_LAYOUT_LIST) {
        if (tid == 0) store_scratch(out_dir, r, e.sz, 0, kFValid);
        return;
    }
    const uint16_t* L = reinterpret_cast<const uint16_t*>(payload + e.off);
    const uint32_t n_c = s_nc;
    uint32_t vb = 0;
    bool bad = false;
    for (uint32_t j = tid; j < e.K; j += kPT) {
        const uint32_t cur = L[j];
        uint32_t gap = cur;
        if (j) {
            const uint32_t prv = L[j - 1];
            bad |= prv >= cur;
            gap = cur - prv - 1u;
        }
        bad |= cur >= n_c;
        vb += leb_len(gap);
    }
    if (bad) s_bad = 1;   // benign race: every writer stores 1
    uint32_t total = 0;
    (void)block_scan32(vb, total, sh);
    if (tid == 0) {
        if (s_bad) {
            atomicOr(ctr + kPkErr, kErrFormat);
            store_scratch(out_dir, r, 0, 0, 0);
        } else if (p16(total) < p16(2 * e.K)) {
            store_scratch(out_dir, r, p16(total) + e.sz - p16(2 * e.K), total, kFValid | kFGaps);
        } else {
            store_scratch(out_dir, r, e.sz, 0, kFValid);
        }
    }
}

// Unpacking: one thread per record.  The unpacked size of a gap record
// follows from its entry alone (an index list of K changes); the gap section
// must be a multiple of 16 bytes and strictly smaller than that list.  Each
// record must start where the previous one ends.
__global__ __launch_bounds__(256) void up_size_kernel(const DevTensor* tensors, uint32_t n_tensors, const uint8_t* dir,
                                                      uint64_t n, uint64_t payload_bytes, uint8_t* out_dir,
                                                      unsigned long long* ctr) {
    const uint64_t r = uint64_t(blockIdx.x) * 256u + threadIdx.x;
    if (r >= n) return;
    const Ent e = load_ent(dir, r);
    const uint32_t n_c = entry_n_c(tensors, n_tensors, e.t, e.c, e.w);
    bool ok = n_c != 0 && (e.off & 15u) == 0 && e.off <= payload_bytes && e.sz <= payload_bytes - e.off;
    uint64_t prev_end = 0;
    if (r) {
        const Ent p = load_ent(dir, r - 1);
        prev_end = p.off + p.sz;
    }
    ok = ok && e.off == prev_end && (r + 1 < n || e.off + e.sz == payload_bytes);
    uint64_t size = 0;
    uint32_t sec = 0, flags = 0;
    if (ok && e.layout == DCR_LAYOUT_GAPS) {
        const uint32_t full = record_bytes(e.w, n_c, e.K, e.kind, e.hm, e.H, DCR_LAYOUT_LIST);
        const uint32_t tail = full - p16(2 * e.K);
        ok = full != 0 && e.sz > tail;
        sec = ok ? e.sz - tail : 0u;
        ok = ok && (sec & 15u) == 0 && sec < p16(2 * e.K);
        size = full;
        flags = kFValid | kFGaps;
    } else if (ok) {
        ok = e.layout <= DCR_LAYOUT_LIST && record_bytes(e.w, n_c, e.K, e.kind, e.hm, e.H, e.layout) == e.sz;
        size = e.sz;
        flags = kFValid;
    }
    if (!ok) {
        atomicOr(ctr + kPkErr, kErrFormat);
        size = sec = flags = 0;
    }
    store_scratch(out_dir, r, size, sec, flags);
}

// ----------------------------------------------------------------- scan

// Exclusive scan of one 64-bit value per thread of a kST workgroup.
__device__ uint64_t scan1024(uint64_t v, uint64_t& total, uint64_t* sh) {
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    uint64_t x = v;
#pragma unroll
    for (uint32_t d = 1; d < 64; d <<= 1) {
        const uint64_t y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) sh[wave] = x;
    __syncthreads();
    uint64_t pre = 0, tot = 0;
#pragma unroll
    for (uint32_t w = 0; w < kST / 64; w++) {
        pre += w < wave ? sh[w] : 0;
        tot += sh[w];
    }
    __syncthreads();
    total = tot;
    return pre + x - v;
}

__device__ __forceinline__ uint64_t slot_size(const uint8_t* dir, uint64_t r) {
    return *reinterpret_cast<const uint64_t*>(dir + r * DCR_DIRENT_BYTES);
}

// Sum of the sizes of records [b * kST, (b + 1) * kST).
__global__ __launch_bounds__(kST) void pk_reduce_kernel(const uint8_t* out_dir, uint64_t n, uint64_t* bsum) {
    __shared__ uint64_t sh[kST / 64];
    const uint64_t r = uint64_t(blockIdx.x) * kST + threadIdx.x;
    uint64_t total = 0;
    (void)scan1024(r < n ? slot_size(out_dir, r) : 0, total, sh);
    if (threadIdx.x == 0) bsum[blockIdx.x] = total;
}

// Exclusive scan of the nb block sums, in place; the grand total to ctr.
__global__ __launch_bounds__(kST) void pk_scan_sums_kernel(uint64_t* bsum, uint64_t nb, unsigned long long* ctr) {
    __shared__ uint64_t sh[kST / 64];
    uint64_t carry = 0;
    for (uint64_t base = 0; base < nb; base += kST) {
        const uint64_t i = base + threadIdx.x;
        const uint64_t v = i < nb ? bsum[i] : 0;
        uint64_t total = 0;
        const uint64_t ex = scan1024(v, total, sh);
        if (i < nb) bsum[i] = carry + ex;
        carry += total;
    }
    if (threadIdx.x == 0) ctr[kPkTotal] = carry;
}

// Each record's output offset (scratch word 1).
__global__ __launch_bounds__(kST) void pk_downsweep_kernel(uint8_t* out_dir, uint64_t n, const uint64_t* bsum) {
    __shared__ uint64_t sh[kST / 64];
    const uint64_t r = uint64_t(blockIdx.x) * kST + threadIdx.x;
    uint64_t total = 0;
    const uint64_t ex = scan1024(r < n ? slot_size(out_dir, r) : 0, total, sh);
    if (r < n) *reinterpret_cast<uint64_t*>(out_dir + r * DCR_DIRENT_BYTES + 8) = bsum[blockIdx.x] + ex;
}

// ---------------------------------------------------------------- write

struct Slot {
    uint64_t size, off;
    uint32_t sec, flags;
};

__device__ __forceinline__ Slot load_slot(const uint8_t* dir, uint64_t r) {
    const uint4* p = reinterpret_cast<const uint4*>(dir + r * DCR_DIRENT_BYTES);
    const uint4 a = p[0], b = p[1];
    return Slot{uint64_t(a.x) | (uint64_t(a.y) << 32), uint64_t(a.z) | (uint64_t(a.w) << 32), b.x, b.y};
}

__device__ __forceinline__ void copy16(uint8_t* dst, const uint8_t* src, uint32_t bytes) {
    for (uint32_t q = threadIdx.x; q < bytes / 16; q += kPT)
        reinterpret_cast<uint4*>(dst)[q] = reinterpret_cast<const uint4*>(src)[q];
}

// Packing: one workgroup per record.  A packed list: thread t writes the
// gap varints of changes [t * per, (t + 1) * per) at the byte position a
// workgroup scan of their lengths gives; then the padding and the later
// sections.  Other records are copied.  Thread 0 then replaces the scratch
// slot with the final entry.
__global__ __launch_bounds__(kPT) void pk_write_kernel(const uint8_t* dir, const uint8_t* payload, uint8_t* out_dir,
                                                       uint8_t* out_payload, uint64_t payload_cap) {
    __shared__ uint32_t sh[kPT / 64];
    __shared__ Slot s_slot;
    const uint64_t r = blockIdx.x;
    const uint32_t tid = threadIdx.x;
    if (tid == 0) s_slot = load_slot(out_dir, r);
    __syncthreads();
    const Slot sl = s_slot;
    if (!(sl.flags & kFValid) || sl.off + sl.size > payload_cap) return;   // uniform; status set at the end
    Ent e = load_ent(dir, r);
    const uint8_t* src = payload + e.off;
    uint8_t* dst = out_payload + sl.off;
    if (sl.flags & kFGaps) {
        const uint16_t* L = reinterpret_cast<const uint16_t*>(src);
        const uint32_t per = (e.K + kPT - 1) / kPT, j0 = min(e.K, tid * per), j1 = min(e.K, j0 + per);
        uint32_t mine = 0;
        for (uint32_t j = j0; j < j1; j++) mine += leb_len(j ? uint32_t(L[j]) - L[j - 1] - 1u : uint32_t(L[j]));
        uint32_t total = 0;
        uint32_t pos = block_scan32(mine, total, sh);
        for (uint32_t j = j0; j < j1; j++) {
            uint32_t v = j ? uint32_t(L[j]) - L[j - 1] - 1u : uint32_t(L[j]);
            while (v >= 0x80u) {
                dst[pos++] = uint8_t((v & 0x7Fu) | 0x80u);
                v >>= 7;
            }
            dst[pos++] = uint8_t(v);
        }
        for (uint32_t q = sl.sec + tid; q < p16(sl.sec); q += kPT) dst[q] = 0;
        copy16(dst + p16(sl.sec), src + p16(2 * e.K), e.sz - p16(2 * e.K));
        e.layout = DCR_LAYOUT_GAPS;
    } else {
        copy16(dst, src, e.sz);
    }
    __syncthreads();
    if (tid == 0) {
        e.off = sl.off;
        e.sz = uint32_t(sl.size);
        store_ent(out_dir, r, e);
    }
}

// Unpacking: one workgroup per record.  A gap record: thread t takes bytes
// [t * per, (t + 1) * per) of the gap section and counts the varints ending
// there (bytes with the high bit clear); a scan numbers them.  Each such
// varint is read back from its last byte (at most three bytes, the last one
// nonzero unless it is the only one, a value below 2^16); a second scan of
// the gaps plus one gives every index, written as a 16-bit list.  Exactly K
// varints, zero bytes after the K-th, and the last index below the chunk's
// elements, or the stream is refused.
__global__ __launch_bounds__(kPT) void up_write_kernel(const DevTensor* tensors, uint32_t n_tensors, const uint8_t* dir,
                                                       const uint8_t* payload, uint8_t* out_dir, uint8_t* out_payload,
                                                       uint64_t payload_cap, unsigned long long* ctr) {
    __shared__ uint32_t sh[kPT / 64];
    __shared__ Slot s_slot;
    __shared__ uint32_t s_endK, s_bad;
    const uint64_t r = blockIdx.x;
    const uint32_t tid = threadIdx.x;
    if (tid == 0) {
        s_slot = load_slot(out_dir, r);
        s_endK = 0xFFFFFFFFu;
        s_bad = 0;
    }
    __syncthreads();
    const Slot sl = s_slot;
    if (!(sl.flags & kFValid) || sl.off + sl.size > payload_cap) return;   // uniform
    Ent e = load_ent(dir, r);
    const uint8_t* src = payload + e.off;
    uint8_t* dst = out_payload + sl.off;
    if (sl.flags & kFGaps) {
        const uint32_t K = e.K, sec = sl.sec;
        const uint32_t n_c = entry_n_c(tensors, n_tensors, e.t, e.c, e.w);
        const uint32_t per = (sec + kPT - 1) / kPT, b0 = min(sec, tid * per), b1 = min(sec, b0 + per);
        uint32_t nterm = 0;
        for (uint32_t b = b0; b < b1; b++) nterm += src[b] < 0x80u ? 1u : 0u;
        uint32_t tterm = 0;
        const uint32_t tbase = block_scan32(nterm, tterm, sh);
        bool bad = tterm < K;   // a varint cut off by the section's end
        // this thread's values: gaps + 1, summed
        uint32_t gsum = 0;
        uint32_t i = tbase;
        for (uint32_t b = b0; b < b1; b++) {
            if (src[b] >= 0x80u) continue;
            if (i < K) {
                uint32_t s = b;
                while (s > 0 && src[s - 1] >= 0x80u && b - s < 3) s--;
                if (s > 0 && src[s - 1] >= 0x80u) bad = true;          // more than three bytes
                uint32_t v = 0;
                for (uint32_t q = b + 1; q-- > s;) v = (v << 7) | (src[q] & 0x7Fu);
                if (b > s && src[b] == 0) bad = true;                   // not minimal
                if (v > 0xFFFFu) bad = true;
                gsum += v + 1u;
                if (i == K - 1) s_endK = b;
            }
            i++;
        }
        uint32_t gtot = 0;
        const uint32_t gbase = block_scan32(gsum, gtot, sh);   // its barriers publish s_endK
        const uint32_t endK = s_endK;
        // zero bytes after the K-th varint
        for (uint32_t b = b0; b < b1; b++)
            if (b > endK && src[b] != 0) bad = true;
        if (tterm >= K && gtot - 1u >= n_c) bad = true;        // the last index
        // the indices, as a 16-bit list
        uint32_t run = gbase;
        i = tbase;
        uint16_t* out16 = reinterpret_cast<uint16_t*>(dst);
        for (uint32_t b = b0; b < b1; b++) {
            if (src[b] >= 0x80u) continue;
            if (i < K) {
                uint32_t s = b;
                while (s > 0 && src[s - 1] >= 0x80u && b - s < 3) s--;
                uint32_t v = 0;
                for (uint32_t q = b + 1; q-- > s;) v = (v << 7) | (src[q] & 0x7Fu);
                run += v + 1u;
                out16[i] = uint16_t(run - 1u);
            }
            i++;
        }
        for (uint32_t q = 2 * K + tid; q < p16(2 * K); q += kPT) dst[q] = 0;
        copy16(dst + p16(2 * K), src + sec, e.sz - sec);
        if (bad) s_bad = 1;   // benign race: every writer stores 1
        e.layout = DCR_LAYOUT_LIST;
    } else {
        copy16(dst, src, e.sz);
    }
    __syncthreads();
    if (tid == 0) {
        if (s_bad) atomicOr(ctr + kPkErr, kErrFormat);
        e.off = sl.off;
        e.sz = uint32_t(sl.size);
        store_ent(out_dir, r, e);
    }
}

// Header (the input's, with the other magic and the new payload size) and result.
__global__ void pk_finish_kernel(const unsigned long long* ctr, dcr_stream_header hdr, uint32_t magic, uint64_t n,
                                 uint64_t payload_cap, dcr_stream_header* out_hdr, dcr_encode_result* res) {
    if (threadIdx.x != 0) return;
    const uint64_t total = ctr[kPkTotal];
    const bool bad = ctr[kPkErr] != 0;
    hdr.magic = magic;
    hdr.payload_bytes = bad ? 0 : total;
    *out_hdr = hdr;
    dcr_encode_result r;
    r.n_records = n;
    r.payload_bytes = total;
    r.n_changed = 0;
    r.status = bad ? DCR_E_FORMAT : (total > payload_cap ? DCR_E_CAPACITY : DCR_OK);
    r.n_reencoded = 0;
    *res = r;
}

int32_t fail(int32_t rc, const std::string& m) {
    set_error(m);
    return rc;
}
bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared host path of both directions.
int32_t transport(const dcr_plan* plan, const dcr_stream_header* h, const void* dir_dev, const void* payload_dev,
                  void* header_out, void* dir_out, uint64_t dir_cap, void* payload_out, uint64_t payload_cap,
                  dcr_encode_result* result_dev, void* workspace_dev, uint64_t ws_bytes, void* stream, bool pack) {
    if (!plan) return fail(DCR_E_INVAL, "plan is NULL");
    const Plan& p = *plan;
    if (!p.dev_tables) return fail(DCR_E_INVAL, "plan not uploaded");
    if (!h) return fail(DCR_E_INVAL, "header is NULL");
    const uint32_t want_magic = pack ? DCR_MAGIC : kMagicPacked;
    if (h->magic != want_magic || h->format_version != DCR_FORMAT_VERSION || h->chunk_bytes != DCR_CHUNK_BYTES ||
        h->reserved0 != 0 || h->reserved1 != 0 || h->stream_kind > DCR_MODE_RETRY)
        return fail(DCR_E_FORMAT, pack ? "stream header: not a plain stream (magic / version / chunk size / kind)"
                                       : "stream header: not a packed stream (magic / version / chunk size / kind)");
    if (h->plan_fingerprint != p.fingerprint) return fail(DCR_E_FORMAT, "stream header: plan fingerprint mismatch");
    const uint64_t n = h->n_records;
    if (n > 2 * uint64_t(p.chunks.size()))
        return fail(DCR_E_FORMAT, "stream header: more records than two per chunk of the plan");
    if (n && (!dir_dev || !payload_dev)) return fail(DCR_E_INVAL, "NULL stream buffer");
    if (!header_out || !result_dev || !workspace_dev || (n && !dir_out) || (payload_cap && !payload_out))
        return fail(DCR_E_INVAL, "NULL output buffer");
    if (!al16(dir_dev) || !al16(payload_dev) || !al16(header_out) || !al16(dir_out) || !al16(payload_out) ||
        !al16(result_dev) || !al16(workspace_dev))
        return fail(DCR_E_INVAL, "buffer not 16-byte aligned");
    if (dir_cap < n * DCR_DIRENT_BYTES)
        return fail(DCR_E_CAPACITY, "output directory smaller than n_records entries");
    if (ws_bytes < p.ws_bytes) return fail(DCR_E_CAPACITY, "workspace too small");
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace_dev);
    auto* ctr = reinterpret_cast<unsigned long long*>(ws + p.ws_counter);
    auto* bsum = reinterpret_cast<uint64_t*>(ws + p.ws_status);   // n_tiles words >= the block count
    const auto* tensors = reinterpret_cast<const DevTensor*>(static_cast<const uint8_t*>(p.dev_tables) + p.off_tensors);
    const uint32_t nT = uint32_t(p.tensors.size());
    const auto* d_in = static_cast<const uint8_t*>(dir_dev);
    const auto* p_in = static_cast<const uint8_t*>(payload_dev);
    auto* d_out = static_cast<uint8_t*>(dir_out);
    auto* p_out = static_cast<uint8_t*>(payload_out);
    const uint64_t nb = (n + kST - 1) / kST;
    hipLaunchKernelGGL(pk_clear_kernel, dim3(1), dim3(64), 0, st, ctr);
    if (n) {
        if (pack)
            hipLaunchKernelGGL(pk_size_kernel, dim3(uint32_t(n)), dim3(kPT), 0, st, tensors, nT, d_in, p_in,
                               h->payload_bytes, d_out, ctr);
        else
            hipLaunchKernelGGL(up_size_kernel, dim3(uint32_t((n + 255) / 256)), dim3(256), 0, st, tensors, nT, d_in,
                               n, h->payload_bytes, d_out, ctr);
        hipLaunchKernelGGL(pk_reduce_kernel, dim3(uint32_t(nb)), dim3(kST), 0, st, d_out, n, bsum);
    }
    hipLaunchKernelGGL(pk_scan_sums_kernel, dim3(1), dim3(kST), 0, st, bsum, nb, ctr);
    if (n) {
        hipLaunchKernelGGL(pk_downsweep_kernel, dim3(uint32_t(nb)), dim3(kST), 0, st, d_out, n, bsum);
        if (pack)
            hipLaunchKernelGGL(pk_write_kernel, dim3(uint32_t(n)), dim3(kPT), 0, st, d_in, p_in, d_out, p_out,
                               payload_cap);
        else
            hipLaunchKernelGGL(up_write_kernel, dim3(uint32_t(n)), dim3(kPT), 0, st, tensors, nT, d_in, p_in, d_out,
                               p_out, payload_cap, ctr);
    }
    hipLaunchKernelGGL(pk_finish_kernel, dim3(1), dim3(64), 0, st, ctr, *h, pack ? kMagicPacked : DCR_MAGIC, n,
                       payload_cap, static_cast<dcr_stream_header*>(header_out), result_dev);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(DCR_E_HIP, std::string("launch: ") + hipGetErrorString(e));
    return DCR_OK;
}

}  // namespace
}  // namespace dcr

extern "C" {

int32_t dcr_stream_pack(const dcr_plan* plan, const dcr_stream_header* header, const void* dir_dev,
                        const void* payload_dev, void* header_out_dev, void* dir_out_dev, uint64_t dir_cap,
                        void* payload_out_dev, uint64_t payload_cap, dcr_encode_result* result_dev,
                        void* workspace_dev, uint64_t ws_bytes, void* stream) {
    dcr::set_error("");
    return dcr::transport(plan, header, dir_dev, payload_dev, header_out_dev, dir_out_dev, dir_cap, payload_out_dev,
                          payload_cap, result_dev, workspace_dev, ws_bytes, stream, true);
}

int32_t dcr_stream_unpack(const dcr_plan* plan, const dcr_stream_header* header, const void* dir_dev,
                          const void* payload_dev, void* header_out_dev, void* dir_out_dev, uint64_t dir_cap,
                          void* payload_out_dev, uint64_t payload_cap, dcr_encode_result* result_dev,
                          void* workspace_dev, uint64_t ws_bytes, void* stream) {
    dcr::set_error("");
    return dcr::transport(plan, header, dir_dev, payload_dev, header_out_dev, dir_out_dev, dir_cap, payload_out_dev,
                          payload_cap, result_dev, workspace_dev, ws_bytes, stream, false);
}

}  // extern "C"
