// dcr_plan.cpp -- host side of libdcr.so: the direct-projection plan.
//
// A plan turns the trainer layout (affine segments: shard-local index ->
// canonical checkpoint coordinate, ai-feeds summary "key modules" 1; ai.info
// abstract) into the tables the gfx950 kernels read: one entry per 64 KiB
// canonical chunk and, per chunk, the contiguous shard runs ("pieces") that
// fill it, in canonical order.  Like the CPU-prepared tiling / address plan of
// the humansand page ("A strong baseline with Blackwell-native DE"), all of
// this metadata is built once per layout on the host.  The build also checks
// the ownership invariant: every canonical element covered exactly once (the
// tokendh blog's one owner per shard; the humansand page's exactly-once
// ownership remap).
#include <algorithm>
#include <cstring>
#include <new>

#include "dcr_internal.h"

namespace dcr {

static thread_local std::string g_err;
void set_error(const std::string& msg) { g_err = msg; }

static uint64_t pad16(uint64_t x) { return (x + 15) & ~uint64_t(15); }
static uint64_t pad256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

struct Run {
    uint64_t canon;      // canonical element index
    uint64_t shard_off;  // shard element index
    uint64_t len;
    uint32_t shard;
};

static int32_t fail(int32_t rc, const std::string& msg) {
    set_error(msg);
    return rc;
}

static int32_t check_tensor(const dcr_tensor_desc* T, uint32_t nT, uint32_t t) {
    const dcr_tensor_desc& d = T[t];
    const uint32_t w = d.elem_bytes;
    const std::string id = "tensor " + std::to_string(t) + ": ";
    if (w != 1 && w != 2 && w != 4) return fail(DCR_E_INVAL, id + "elem_bytes must be 1, 2 or 4");
    if (d.route > DCR_ROUTE_BLOCK_SCALED) return fail(DCR_E_INVAL, id + "bad route");
    if (d.route != DCR_ROUTE_OVERWRITE && w == 4)
        return fail(DCR_E_INVAL, id + "XOR-carrying routes need 1- or 2-byte elements");
    if (d.numel > (uint64_t(1) << 46)) return fail(DCR_E_INVAL, id + "numel too large");
    if (d.route == DCR_ROUTE_BLOCK_SCALED) {
        if (d.scale_tensor < 0 || uint32_t(d.scale_tensor) >= nT || uint32_t(d.scale_tensor) == t)
            return fail(DCR_E_INVAL, id + "bad scale_tensor");
        const dcr_tensor_desc& s = T[d.scale_tensor];
        if (s.elem_bytes != 4 || s.route != DCR_ROUTE_OVERWRITE)
            return fail(DCR_E_INVAL, id + "scale tensor must be fp32 OVERWRITE");
        if (d.scale_block == 0 || d.scale_block % (16u / w) != 0)
            return fail(DCR_E_INVAL, id + "scale_block must be a positive multiple of 16/elem_bytes");
        if (s.numel != (d.numel + d.scale_block - 1) / d.scale_block)
            return fail(DCR_E_INVAL, id + "scale tensor numel != ceil(numel / scale_block)");
    } else if (d.scale_tensor != -1 || d.scale_block != 0) {
        return fail(DCR_E_INVAL, id + "scale_tensor / scale_block set on a non block-scaled tensor");
    }
    return DCR_OK;
}

// Expand one segment into contiguous runs (after bounds checks).
static int32_t expand_segment(const dcr_segment& g, uint32_t w, uint64_t numel, uint64_t shard_bytes,
                              uint64_t seg_index, std::vector<Run>& out, uint64_t& covered) {
    const std::string id = "segment " + std::to_string(seg_index) + ": ";
    const uint32_t nd = g.ndim;
    if (nd < 1 || nd > 4) return fail(DCR_E_INVAL, id + "ndim must be 1..4");
    unsigned __int128 total = 1;
    for (uint32_t k = 0; k < nd; k++) total *= g.extent[k];
    if (total == 0) return DCR_OK;
    if (total > numel || covered + uint64_t(total) > numel)
        return fail(DCR_E_COVERAGE, id + "covers more elements than the tensor has");
    // bounds of the canonical and the shard index over the whole segment
    __int128 cmin = g.canon_off, cmax = g.canon_off, smin = g.shard_off, smax = g.shard_off;
    for (uint32_t k = 0; k < nd; k++) {
        if (g.extent[k] > (uint64_t(1) << 46)) return fail(DCR_E_INVAL, id + "extent too large");
        const __int128 ce = __int128(g.extent[k] - 1) * g.canon_stride[k];
        const __int128 se = __int128(g.extent[k] - 1) * g.shard_stride[k];
        (ce < 0 ? cmin : cmax) += ce;
        (se < 0 ? smin : smax) += se;
    }
    if (cmin < 0 || cmax >= __int128(numel)) return fail(DCR_E_INVAL, id + "canonical index out of range");
    if (smin < 0 || (smax + 1) * w > __int128(shard_bytes))
        return fail(DCR_E_INVAL, id + "shard index out of range");
    covered += uint64_t(total);
    // innermost dimension contiguous in both spaces -> runs of extent[nd-1]
    const uint32_t last = nd - 1;
    const bool inner = g.canon_stride[last] == 1 && g.shard_stride[last] == 1;
    const uint32_t outer_dims = inner ? last : nd;
    const uint64_t run_len = inner ? g.extent[last] : 1;
    uint64_t x[4] = {0, 0, 0, 0};
    uint64_t n_outer = uint64_t(total) / run_len;
    for (uint64_t i = 0; i < n_outer; i++) {
        int64_t c = int64_t(g.canon_off), s = int64_t(g.shard_off);
        for (uint32_t k = 0; k < outer_dims; k++) {
            c += int64_t(x[k]) * g.canon_stride[k];
            s += int64_t(x[k]) * g.shard_stride[k];
        }
        if (!out.empty()) {
            Run& p = out.back();
            if (p.shard == g.shard_id && p.canon + p.len == uint64_t(c) && p.shard_off + p.len == uint64_t(s)) {
                p.len += run_len;
                goto next;
            }
        }
        out.push_back(Run{uint64_t(c), uint64_t(s), run_len, g.shard_id});
    next:
        for (uint32_t k = outer_dims; k-- > 0;) {
            if (++x[k] < g.extent[k]) break;
            x[k] = 0;
        }
    }
    return DCR_OK;
}

static uint64_t fnv1a64(const dcr_tensor_desc* T, uint32_t nT) {
    uint64_t h = 0xcbf29ce484222325ull;
    for (uint32_t t = 0; t < nT; t++) {
        uint8_t rec[24];
        auto put = [&](int off, uint64_t v, int n) {
            for (int i = 0; i < n; i++) rec[off + i] = uint8_t(v >> (8 * i));
        };
        put(0, T[t].numel, 8);
        put(8, T[t].elem_bytes, 4);
        put(12, T[t].route, 4);
        put(16, uint32_t(T[t].scale_tensor), 4);
        put(20, T[t].scale_block, 4);
        for (int i = 0; i < 24; i++) {
            h ^= rec[i];
            h *= 0x100000001b3ull;
        }
    }
    return h;
}

static int32_t build(const dcr_tensor_desc* T, uint32_t nT, const uint64_t* shard_bytes, uint32_t nS,
                     const dcr_segment* segs, uint64_t nseg, Plan& P) {
    for (uint32_t t = 0; t < nT; t++) {
        int32_t rc = check_tensor(T, nT, t);
        if (rc) return rc;
    }
    P.tensors.assign(T, T + nT);
    P.shard_bytes.assign(shard_bytes, shard_bytes + nS);

    // segments grouped by tensor
    std::vector<uint64_t> order(nseg);
    for (uint64_t i = 0; i < nseg; i++) {
        if (segs[i].tensor_id >= nT) return fail(DCR_E_INVAL, "segment " + std::to_string(i) + ": bad tensor_id");
        if (segs[i].shard_id >= nS) return fail(DCR_E_INVAL, "segment " + std::to_string(i) + ": bad shard_id");
        order[i] = i;
    }
    std::stable_sort(order.begin(), order.end(),
                     [&](uint64_t a, uint64_t b) { return segs[a].tensor_id < segs[b].tensor_id; });

    P.dt.resize(nT);
    uint64_t seg_pos = 0;
    std::vector<Run> runs;
    std::vector<uint8_t> is_scale_used(nT, 0);
    uint32_t widths = 0;   // the element widths of the chunks, OR-ed
    for (uint32_t t = 0; t < nT; t++) {
        const dcr_tensor_desc& d = T[t];
        const uint32_t w = d.elem_bytes;
        const uint64_t E = kChunkBytes / w;
        runs.clear();
        uint64_t covered = 0;
        for (; seg_pos < nseg && segs[order[seg_pos]].tensor_id == t; seg_pos++) {
            const dcr_segment& g = segs[order[seg_pos]];
            int32_t rc = expand_segment(g, w, d.numel, shard_bytes[g.shard_id], order[seg_pos], runs, covered);
            if (rc) return rc;
        }
        std::sort(runs.begin(), runs.end(), [](const Run& a, const Run& b) { return a.canon < b.canon; });
        uint64_t cursor = 0;
        size_t m = 0;
        for (size_t i = 0; i < runs.size(); i++) {
            if (runs[i].canon != cursor)
                return fail(DCR_E_COVERAGE, "tensor " + std::to_string(t) + ": canonical element " +
                                                std::to_string(std::min(cursor, runs[i].canon)) +
                                                (runs[i].canon > cursor ? " not covered" : " covered twice"));
            cursor += runs[i].len;
            if (m > 0 && runs[m - 1].shard == runs[i].shard &&
                runs[m - 1].shard_off + runs[m - 1].len == runs[i].shard_off) {
                runs[m - 1].len += runs[i].len;
            } else {
                runs[m++] = runs[i];
            }
        }
        runs.resize(m);
        if (cursor != d.numel)
            return fail(DCR_E_COVERAGE, "tensor " + std::to_string(t) + ": canonical element " +
                                            std::to_string(cursor) + " not covered");
        const uint64_t nch = (d.numel + E - 1) / E;
        if (P.chunks.size() + nch > kMaxTiles)
            return fail(DCR_E_INVAL, "plan has more than " + std::to_string(kMaxTiles) +
                                         " chunks (one encode workgroup per chunk in one grid)");
        DevTensor& dt = P.dt[t];
        dt = DevTensor{};
        dt.numel = d.numel;
        dt.w = w;
        dt.route = d.route;
        dt.n_chunks = uint32_t(nch);
        dt.scale_tensor = d.scale_tensor;
        dt.scale_block = d.scale_block;
        dt.first_chunk = uint32_t(P.chunks.size());
        size_t ri = 0;
        for (uint64_t c = 0; c < nch; c++) {
            const uint64_t c0 = c * E, c1 = std::min(d.numel, c0 + E);
            DevChunk ch{t, uint32_t(c), uint32_t(P.pieces.size()), 0};
            while (ri < runs.size() && runs[ri].canon + runs[ri].len <= c0) ri++;
            for (size_t rj = ri; rj < runs.size() && runs[rj].canon < c1; rj++) {
                const uint64_t a = std::max(c0, runs[rj].canon);
                const uint64_t b = std::min(c1, runs[rj].canon + runs[rj].len);
                DevPiece p;
                p.shard_elem_off = runs[rj].shard_off + (a - runs[rj].canon);
                p.shard = runs[rj].shard;
                p.canon_start = uint16_t(a - c0);
                p.len_m1 = uint16_t(b - a - 1);
                P.pieces.push_back(p);
                ch.n_pieces++;
            }
            if (P.pieces.size() > 0xFFFFFFFFull) return fail(DCR_E_INVAL, "plan has too many pieces");
            // direct: each 16-byte group sits inside one piece at a 16-byte
            // aligned shard offset (shard bases are 16-byte aligned)
            const uint32_t V = 16 / w;
            bool direct = (c1 - c0) % V == 0 && ch.n_pieces <= kMaxCachedPieces;
            for (uint32_t i = 0; direct && i < ch.n_pieces; i++) {
                const DevPiece& pp = P.pieces[ch.first_piece + i];
                direct = pp.canon_start % V == 0 && (uint32_t(pp.len_m1) + 1) % V == 0 && pp.shard_elem_off % V == 0;
            }
            if (direct) {
                ch.n_pieces |= kChunkDirect;
                P.direct[w == 1 ? 0 : (w == 2 ? 1 : 2)].push_back(uint32_t(P.chunks.size()));
            } else {
                P.slow.push_back(uint32_t(P.chunks.size()));
            }
            P.chunks.push_back(ch);
            widths |= w;
            // worst-case stream sizes (DELTA or RETRY, whichever is larger)
            const uint64_t n_c = c1 - c0, nb = pad16((n_c + 7) / 8);
            uint64_t worst = nb + w * pad16(n_c);                       // one dense record
            uint64_t ents = 1;
            if (d.route == DCR_ROUTE_BLOCK_SCALED) {
                worst = std::max(worst, 2 * nb + w * (n_c + 30));         // XOR + OW records
                ents = 2;
            }
            // the chunk's staging slot: its worst case, 16-byte aligned
            P.slots.push_back(P.max_payload_bytes);
            P.max_payload_bytes += pad16(worst);
            P.max_dir_bytes += ents * DCR_DIRENT_BYTES;
        }
        P.canonical_bytes += d.numel * w;
        if (d.route == DCR_ROUTE_BLOCK_SCALED) is_scale_used[d.scale_tensor] = 1;
    }
    // the least staging area the encode uses compactly: 1/16 of the worst
    // case (about 4 KiB a chunk of 2-byte elements, the records of a chunk
    // with ~1 % of its elements changed), and 16 bytes a partition at least
    P.compact_stage_bytes = std::max<uint64_t>(pad16(P.max_payload_bytes / 16), uint64_t(kStageParts) * 16);
    P.widths = widths;   // 1, 2 or 4: one bit each
    // per-block "scale changed" flag bits, one bit per element of each gating scale tensor
    std::vector<uint64_t> bit_off(nT, 0);
    for (uint32_t s = 0; s < nT; s++) {
        if (!is_scale_used[s]) continue;
        bit_off[s] = P.scale_bits;
        P.dt[s].scale_bit_off = P.scale_bits;   // a scale tensor's own flag bits
        P.scale_bits += (T[s].numel + 63) / 64 * 64;
        for (uint32_t c = 0; c < P.dt[s].n_chunks; c++) P.scale_chunks.push_back(P.dt[s].first_chunk + c);
    }
    for (uint32_t t = 0; t < nT; t++)
        if (T[t].route == DCR_ROUTE_BLOCK_SCALED) P.dt[t].scale_bit_off = bit_off[T[t].scale_tensor];
    P.fingerprint = fnv1a64(T, nT);
    // does any shard element hold two canonical elements?  (harmless for a
    // sender, which only reads; a receiver layout must not)
    {
        struct ByteRun { uint32_t shard; uint64_t off, len; };   // in bytes
        std::vector<ByteRun> runs_s;
        runs_s.reserve(P.pieces.size());
        for (const DevChunk& ch : P.chunks) {
            const uint64_t w = P.dt[ch.tensor].w;
            const uint32_t np = ch.n_pieces & kPiecesMask;
            for (uint32_t i = 0; i < np; i++) {
                const DevPiece& pc = P.pieces[ch.first_piece + i];
                runs_s.push_back({pc.shard, pc.shard_elem_off * w, (uint64_t(pc.len_m1) + 1) * w});
            }
        }
        std::sort(runs_s.begin(), runs_s.end(), [](const ByteRun& x, const ByteRun& y) {
            return x.shard != y.shard ? x.shard < y.shard : x.off < y.off;
        });
        P.shard_disjoint = true;
        for (size_t i = 1; i < runs_s.size() && P.shard_disjoint; i++)
            if (runs_s[i].shard == runs_s[i - 1].shard && runs_s[i - 1].off + runs_s[i - 1].len > runs_s[i].off)
                P.shard_disjoint = false;
    }

    // device tables: tensors | chunks | pieces | scale chunk list
    P.off_tensors = 0;
    P.off_chunks = pad256(P.off_tensors + P.dt.size() * sizeof(DevTensor));
    P.off_pieces = pad256(P.off_chunks + P.chunks.size() * sizeof(DevChunk));
    P.off_scale_chunks = pad256(P.off_pieces + P.pieces.size() * sizeof(DevPiece));
    P.off_slots = pad256(P.off_scale_chunks + P.scale_chunks.size() * sizeof(uint32_t) + 4);
    P.off_slow = pad256(P.off_slots + P.slots.size() * sizeof(uint64_t));
    uint64_t end = pad256(P.off_slow + P.slow.size() * sizeof(uint32_t) + 4);
    for (int i = 0; i < 3; i++) {
        P.off_direct[i] = end;
        end = pad256(end + P.direct[i].size() * sizeof(uint32_t) + 4);
    }
    P.table_bytes = end;
    P.blob.assign(P.table_bytes, 0);
    if (!P.dt.empty()) std::memcpy(P.blob.data() + P.off_tensors, P.dt.data(), P.dt.size() * sizeof(DevTensor));
    if (!P.chunks.empty())
        std::memcpy(P.blob.data() + P.off_chunks, P.chunks.data(), P.chunks.size() * sizeof(DevChunk));
    if (!P.pieces.empty())
        std::memcpy(P.blob.data() + P.off_pieces, P.pieces.data(), P.pieces.size() * sizeof(DevPiece));
    if (!P.scale_chunks.empty())
        std::memcpy(P.blob.data() + P.off_scale_chunks, P.scale_chunks.data(),
                    P.scale_chunks.size() * sizeof(uint32_t));
    if (!P.slots.empty())
        std::memcpy(P.blob.data() + P.off_slots, P.slots.data(), P.slots.size() * sizeof(uint64_t));
    if (!P.slow.empty())
        std::memcpy(P.blob.data() + P.off_slow, P.slow.data(), P.slow.size() * sizeof(uint32_t));
    for (int i = 0; i < 3; i++)
        if (!P.direct[i].empty())
            std::memcpy(P.blob.data() + P.off_direct[i], P.direct[i].data(), P.direct[i].size() * sizeof(uint32_t));

    // workspace: tile look-back status (a staged encode keeps its list of
    // tiles to encode again there) | fix-up look-back status | partial
    // retry's wanted-chunk bits | counters | shard pointers | scale flags |
    // canonical pointers | per-tile aggregates | per-tile change counts |
    // apply's list of deferred large records | per-tile staging offsets.
    // Everything before the shard pointers is zeroed at the start of an
    // encode.  Bytes past ws_bytes are the optional staging area of encode.
    const uint64_t n_tiles = P.chunks.size();
    P.ws_status = 0;
    P.ws_fix = pad256(n_tiles * 8);
    P.ws_need = pad256(P.ws_fix + (n_tiles + kFixTiles - 1) / kFixTiles * 8);
    P.ws_counter = pad256(P.ws_need + (n_tiles + 63) / 64 * 8);
    P.ws_old = P.ws_counter + kCtrBytes;
    P.ws_new = pad256(P.ws_old + uint64_t(nS) * 8);
    P.ws_scale = pad256(P.ws_new + uint64_t(nS) * 8);
    P.ws_canon = pad256(P.ws_scale + P.scale_bits / 8);
    P.ws_agg = pad256(P.ws_canon + uint64_t(nT) * 8);
    P.ws_info = pad256(P.ws_agg + n_tiles * 8);
    P.big_cap = P.max_dir_bytes / DCR_DIRENT_BYTES;
    P.ws_big = pad256(P.ws_info + n_tiles * 8);
    P.ws_soff = pad256(P.ws_big + P.big_cap * 4);
    P.ws_bytes = pad256(P.ws_soff + n_tiles * 8);
    return DCR_OK;
}

}  // namespace dcr

extern "C" {

int32_t dcr_plan_build(const dcr_tensor_desc* tensors, uint32_t n_tensors, const uint64_t* shard_bytes,
                       uint32_t n_shards, const dcr_segment* segments, uint64_t n_segments, dcr_plan** out) {
    using namespace dcr;
    set_error("");
    if (!out) return fail(DCR_E_INVAL, "out is NULL");
    *out = nullptr;
    if ((n_tensors && !tensors) || (n_shards && !shard_bytes) || (n_segments && !segments))
        return fail(DCR_E_INVAL, "NULL array with a nonzero count");
    dcr_plan* p = new (std::nothrow) dcr_plan();
    if (!p) return fail(DCR_E_NOMEM, "out of host memory");
    int32_t rc;
    try {
        rc = build(tensors, n_tensors, shard_bytes, n_shards, segments, n_segments, *p);
    } catch (const std::bad_alloc&) {
        rc = fail(DCR_E_NOMEM, "out of host memory");
    }
    if (rc) {
        delete p;
        return rc;
    }
    *out = p;
    return DCR_OK;
}

int32_t dcr_plan_query(const dcr_plan* p, dcr_plan_info* out) {
    using namespace dcr;
    if (!p || !out) return fail(DCR_E_INVAL, "NULL argument");
    out->n_tensors = p->tensors.size();
    out->n_shards = p->shard_bytes.size();
    out->n_chunks = p->chunks.size();
    out->n_pieces = p->pieces.size();
    out->table_bytes = p->table_bytes;
    out->workspace_bytes = p->ws_bytes;
    out->max_dir_bytes = p->max_dir_bytes;
    out->max_payload_bytes = p->max_payload_bytes;
    out->fingerprint = p->fingerprint;
    out->canonical_bytes = p->canonical_bytes;
    out->compact_stage_bytes = p->compact_stage_bytes;
    return DCR_OK;
}

void dcr_plan_destroy(dcr_plan* p) { delete p; }

const char* dcr_last_error(void) { return dcr::g_err.c_str(); }

uint32_t dcr_format_constants(uint32_t* out, uint32_t n) {
    const uint32_t v[10] = {DCR_MAGIC, DCR_FORMAT_VERSION, DCR_CHUNK_BYTES, DCR_HEADER_BYTES, DCR_DIRENT_BYTES,
                            uint32_t(sizeof(dcr_tensor_desc)), uint32_t(sizeof(dcr_segment)),
                            uint32_t(sizeof(dcr_stream_header)), uint32_t(DCR_ENC_INDEX_LISTS),
                            uint32_t(DCR_LAYOUT_LIST)};
    uint32_t k = n < 10 ? n : 10;
    for (uint32_t i = 0; i < k && out; i++) out[i] = v[i];
    return k;
}

}  // extern "C"
