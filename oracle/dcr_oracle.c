/*
 * dcr_oracle.c -- TEST INFRASTRUCTURE ONLY (see dcr_oracle.h).
 *
 * A deliberately plain, single-threaded C99 definition of what the GPU
 * library computes.  Tensor by tensor, it materialises the canonical old and
 * new tensors by walking every affine segment element by element, compares
 * stored bits element by element in ascending canonical order, and writes
 * the records byte by byte.  There is no blocking, vectorisation or fusion.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library; the product path never does.
 */
#include "dcr_oracle.h"

#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- helpers */

static uint64_t pad16(uint64_t x) { return (x + 15u) & ~(uint64_t)15u; }

static void put_u16(uint8_t* p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static void put_u32(uint8_t* p, uint32_t v) { int i; for (i = 0; i < 4; i++) p[i] = (uint8_t)(v >> (8 * i)); }
static void put_u64(uint8_t* p, uint64_t v) { int i; for (i = 0; i < 8; i++) p[i] = (uint8_t)(v >> (8 * i)); }
static uint16_t get_u16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static uint32_t get_u32(const uint8_t* p) {
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}
static uint64_t get_u64(const uint8_t* p) {
    uint64_t v = 0; int i;
    for (i = 7; i >= 0; i--) v = (v << 8) | p[i];
    return v;
}

/* Little-endian stored word of element g of a w-byte-per-element buffer. */
static uint32_t load_word(const uint8_t* buf, uint64_t g, uint32_t w) {
    uint32_t v = 0, b;
    for (b = 0; b < w; b++) v |= (uint32_t)buf[g * w + b] << (8 * b);
    return v;
}
static void store_word(uint8_t* buf, uint64_t g, uint32_t w, uint32_t v) {
    uint32_t b;
    for (b = 0; b < w; b++) buf[g * w + b] = (uint8_t)(v >> (8 * b));
}

static uint64_t chunk_elems(uint32_t w) { return ORC_CHUNK_BYTES / w; }
static uint64_t n_chunks(const orc_tensor* t) {
    uint64_t e = chunk_elems(t->elem_bytes);
    return (t->numel + e - 1) / e;
}

/* ------------------------------------------------------------ fingerprint */

uint64_t orc_fingerprint(const orc_tensor* T, uint32_t nT) {
    uint64_t h = 0xcbf29ce484222325ull;
    uint32_t t; int i;
    uint8_t rec[24];
    for (t = 0; t < nT; t++) {
        put_u64(rec, T[t].numel);
        put_u32(rec + 8, T[t].elem_bytes);
        put_u32(rec + 12, T[t].route);
        put_u32(rec + 16, (uint32_t)T[t].scale_tensor);
        put_u32(rec + 20, T[t].scale_block);
        for (i = 0; i < 24; i++) { h ^= rec[i]; h *= 0x100000001b3ull; }
    }
    return h;
}

/* ----------------------------------------------------- table validation */

static int32_t check_tensors(const orc_tensor* T, uint32_t nT) {
    uint32_t t;
    for (t = 0; t < nT; t++) {
        const orc_tensor* d = &T[t];
        uint32_t w = d->elem_bytes;
        if (w != 1 && w != 2 && w != 4) return ORC_E_INVAL;
        if (d->route > ORC_ROUTE_BLOCK_SCALED) return ORC_E_INVAL;
        /* XOR-carrying routes exist for 1- and 2-byte elements only */
        if (d->route != ORC_ROUTE_OVERWRITE && w == 4) return ORC_E_INVAL;
        if (n_chunks(d) > 0xFFFFFFFFull) return ORC_E_INVAL;
        if (d->route == ORC_ROUTE_BLOCK_SCALED) {
            const orc_tensor* s;
            if (d->scale_tensor < 0 || (uint32_t)d->scale_tensor >= nT) return ORC_E_INVAL;
            if ((uint32_t)d->scale_tensor == t) return ORC_E_INVAL;
            s = &T[d->scale_tensor];
            if (s->elem_bytes != 4 || s->route != ORC_ROUTE_OVERWRITE) return ORC_E_INVAL;
            if (d->scale_block == 0 || d->scale_block % (16u / w) != 0) return ORC_E_INVAL;
            if (s->numel != (d->numel + d->scale_block - 1) / d->scale_block) return ORC_E_INVAL;
        } else {
            if (d->scale_tensor != -1 || d->scale_block != 0) return ORC_E_INVAL;
        }
    }
    return ORC_OK;
}

/* -------------------------------------------------- projection (gather) */

/* Walk every segment of tensor t, element by element, copying shard element
 * e to canonical element c.  seen[] counts how often each canonical element
 * is written: every element must be written exactly once. */
static int32_t gather2(const orc_tensor* T, uint32_t nT,
                       const void* const* sh_a, const void* const* sh_b,
                       const uint64_t* shard_bytes, uint32_t nS,
                       const orc_segment* segs, uint64_t nseg,
                       uint32_t t, uint8_t* out_a, uint8_t* out_b) {
    const orc_tensor* d = &T[t];
    uint32_t w = d->elem_bytes;
    uint64_t s, i;
    uint8_t* seen;
    if (t >= nT) return ORC_E_INVAL;
    seen = (uint8_t*)calloc(d->numel ? d->numel : 1, 1);
    if (!seen) return ORC_E_NOMEM;
    for (s = 0; s < nseg; s++) {
        const orc_segment* g = &segs[s];
        uint64_t x[4] = {0, 0, 0, 0};
        uint32_t nd = g->ndim, k;
        uint64_t total = 1;
        if (g->tensor_id != t) continue;
        if (g->shard_id >= nS || nd < 1 || nd > 4) { free(seen); return ORC_E_INVAL; }
        for (k = 0; k < nd; k++) total *= g->extent[k];
        for (i = 0; i < total; i++) {
            int64_t c = (int64_t)g->canon_off, e = (int64_t)g->shard_off;
            for (k = 0; k < nd; k++) {
                c += (int64_t)x[k] * g->canon_stride[k];
                e += (int64_t)x[k] * g->shard_stride[k];
            }
            if (c < 0 || (uint64_t)c >= d->numel) { free(seen); return ORC_E_INVAL; }
            if (e < 0 || ((uint64_t)e + 1) * w > shard_bytes[g->shard_id]) { free(seen); return ORC_E_INVAL; }
            if (seen[c]) { free(seen); return ORC_E_COVERAGE; }
            seen[c] = 1;
            memcpy(out_a + (uint64_t)c * w, (const uint8_t*)sh_a[g->shard_id] + (uint64_t)e * w, w);
            if (out_b)
                memcpy(out_b + (uint64_t)c * w, (const uint8_t*)sh_b[g->shard_id] + (uint64_t)e * w, w);
            /* odometer over the multi-index, last dimension fastest */
            for (k = nd; k-- > 0;) {
                if (++x[k] < g->extent[k]) break;
                x[k] = 0;
            }
        }
    }
    for (i = 0; i < d->numel; i++)
        if (!seen[i]) { free(seen); return ORC_E_COVERAGE; }
    free(seen);
    return ORC_OK;
}

int32_t orc_gather(const orc_tensor* T, uint32_t nT,
                   const void* const* shards, const uint64_t* shard_bytes, uint32_t nS,
                   const orc_segment* segs, uint64_t nseg, uint32_t t, void* out) {
    int32_t rc = check_tensors(T, nT);
    if (rc) return rc;
    if (t >= nT) return ORC_E_INVAL;
    return gather2(T, nT, shards, NULL, shard_bytes, nS, segs, nseg, t, (uint8_t*)out, NULL);
}

/* ---------------------------------------------------------- record bytes */

/* High-byte mode of an XOR record on 2-byte elements with K changes of
 * which h have a nonzero high byte. */
static uint32_t xor_hi_mode(uint64_t K, uint64_t h) {
    if (h == 0) return ORC_HI_NONE;
    if (pad16((K + 7) / 8) + pad16(h) < pad16(K)) return ORC_HI_SPARSE;
    return ORC_HI_DENSE;
}

/* Bytes of a record's first section: the change bitmap (one bit per chunk
 * element), or in the index-list layout K 16-bit element indices; padded. */
static uint64_t head_bytes(uint64_t n_c, uint64_t K, uint32_t layout) {
    return layout == ORC_LAYOUT_LIST ? pad16(2 * K) : pad16((n_c + 7) / 8);
}

/* Layout of a record with K changes: the index list when allowed and
 * strictly smaller than the bitmap. */
static uint32_t choose_layout(uint64_t n_c, uint64_t K, int lists) {
    return (lists && pad16(2 * K) < pad16((n_c + 7) / 8)) ? ORC_LAYOUT_LIST : ORC_LAYOUT_BITMAP;
}

/* Bytes of a record's payload. */
static uint64_t record_bytes(uint64_t n_c, uint32_t w, uint32_t kind, uint64_t K,
                             uint32_t hi_mode, uint64_t H, uint32_t layout) {
    uint64_t sz = head_bytes(n_c, K, layout) + pad16(K);
    if (w == 2 && kind == ORC_KIND_XOR) {
        if (hi_mode == ORC_HI_SPARSE) sz += pad16((K + 7) / 8) + pad16(H);
        else if (hi_mode == ORC_HI_DENSE) sz += pad16(K);
    } else if (w == 2) {
        sz += pad16(K);
    } else if (w == 4) {
        sz += 3 * pad16(K);
    }
    return sz;
}

/* Build one record: idx[j] is the chunk-relative index of change j (ascending),
 * word[j] its w-byte payload word (old^new for XOR, new for OW).  Writes to
 * out (if non-NULL) and returns the byte size; fills hi_mode and H. */
static uint64_t build_record(uint8_t* out, uint64_t n_c, uint32_t w, uint32_t kind,
                             uint64_t K, const uint32_t* idx, const uint32_t* word,
                             uint32_t layout, uint32_t* hi_mode, uint32_t* H) {
    uint64_t j, h = 0, pos, sz;
    uint32_t mode;
    if (w == 2 && kind == ORC_KIND_XOR) {
        for (j = 0; j < K; j++) if ((word[j] >> 8) & 0xFF) h++;
        mode = xor_hi_mode(K, h);
        *H = (uint32_t)(mode == ORC_HI_SPARSE ? h : (mode == ORC_HI_DENSE ? K : 0));
    } else if (w == 1) {
        mode = ORC_HI_NONE; *H = 0;
    } else {
        mode = ORC_HI_DENSE; *H = (uint32_t)K;
    }
    *hi_mode = mode;
    sz = record_bytes(n_c, w, kind, K, mode, *H, layout);
    if (!out) return sz;
    memset(out, 0, sz);
    if (layout == ORC_LAYOUT_LIST) {
        /* section 1: the chunk indices of the changes, 16-bit little-endian */
        for (j = 0; j < K; j++) put_u16(out + 2 * j, (uint16_t)idx[j]);
    } else {
        /* section 1: change bitmap, bit i of the chunk = byte i/8, bit i%8 */
        for (j = 0; j < K; j++) out[idx[j] / 8] |= (uint8_t)(1u << (idx[j] % 8));
    }
    pos = head_bytes(n_c, K, layout);
    /* section 2: low byte plane */
    for (j = 0; j < K; j++) out[pos + j] = (uint8_t)(word[j] & 0xFF);
    pos += pad16(K);
    if (w == 2 && kind == ORC_KIND_XOR) {
        if (mode == ORC_HI_SPARSE) {
            uint64_t q = 0, hp;
            for (j = 0; j < K; j++)
                if ((word[j] >> 8) & 0xFF) out[pos + j / 8] |= (uint8_t)(1u << (j % 8));
            hp = pos + pad16((K + 7) / 8);
            for (j = 0; j < K; j++)
                if ((word[j] >> 8) & 0xFF) out[hp + q++] = (uint8_t)(word[j] >> 8);
        } else if (mode == ORC_HI_DENSE) {
            for (j = 0; j < K; j++) out[pos + j] = (uint8_t)(word[j] >> 8);
        }
    } else if (w >= 2) {
        uint32_t b;
        for (b = 1; b < w; b++) {
            for (j = 0; j < K; j++) out[pos + j] = (uint8_t)(word[j] >> (8 * b));
            pos += pad16(K);
        }
    }
    return sz;
}

static void put_dirent(uint8_t* p, uint32_t t, uint32_t c, uint32_t K, uint32_t kind,
                       uint32_t hi_mode, uint32_t w, uint64_t off, uint32_t sz, uint32_t H, uint32_t layout) {
    put_u32(p + 0, t);
    put_u32(p + 4, c);
    put_u32(p + 8, K);
    p[12] = (uint8_t)kind;
    p[13] = (uint8_t)hi_mode;
    p[14] = (uint8_t)w;
    p[15] = (uint8_t)layout;
    put_u64(p + 16, off);
    put_u32(p + 24, sz);
    put_u32(p + 28, H);
}

static void put_header(uint8_t* p, uint32_t mode, uint64_t base_v, uint64_t new_v,
                       uint64_t fp, uint64_t nrec, uint64_t pbytes) {
    memset(p, 0, ORC_HEADER_BYTES);
    put_u32(p + 0, ORC_MAGIC);
    put_u16(p + 4, (uint16_t)ORC_FORMAT_VER);
    put_u16(p + 6, (uint16_t)mode);
    put_u32(p + 8, ORC_CHUNK_BYTES);
    put_u64(p + 16, base_v);
    put_u64(p + 24, new_v);
    put_u64(p + 32, fp);
    put_u64(p + 40, nrec);
    put_u64(p + 48, pbytes);
}

/* ----------------------------------------------------------------- encode */

/* The encode proper.  need: NULL (every chunk), or one byte per chunk in
 * (tensor, chunk) order, nonzero for the chunks to encode; the others are
 * treated as unchanged. */
static int32_t encode_chunks(const orc_tensor* T, uint32_t nT,
                             const void* const* old_shards, const void* const* new_shards,
                             const uint64_t* shard_bytes, uint32_t nS,
                             const orc_segment* segs, uint64_t nseg,
                             uint32_t mode, uint64_t base_version, uint64_t new_version,
                             uint8_t* header_out,
                             uint8_t* dir_out, uint64_t dir_cap, uint64_t* dir_bytes,
                             uint8_t* payload_out, uint64_t payload_cap, uint64_t* payload_bytes,
                             const uint8_t* need) {
    uint64_t nrec = 0, poff = 0, ordinal = 0;
    uint32_t t;
    int32_t rc = check_tensors(T, nT);
    uint32_t* idx[2] = {NULL, NULL};
    uint32_t* word[2] = {NULL, NULL};
    const int lists = (mode & ORC_ENC_LISTS) != 0;
    if (rc) return rc;
    mode &= ~(uint32_t)ORC_ENC_LISTS;
    if (mode != ORC_MODE_DELTA && mode != ORC_MODE_RETRY) return ORC_E_INVAL;
    idx[0] = (uint32_t*)malloc(65536 * sizeof(uint32_t));
    idx[1] = (uint32_t*)malloc(65536 * sizeof(uint32_t));
    word[0] = (uint32_t*)malloc(65536 * sizeof(uint32_t));
    word[1] = (uint32_t*)malloc(65536 * sizeof(uint32_t));
    if (!idx[0] || !idx[1] || !word[0] || !word[1]) { rc = ORC_E_NOMEM; goto done; }

    for (t = 0; t < nT; t++) {
        const orc_tensor* d = &T[t];
        uint32_t w = d->elem_bytes;
        uint64_t E = chunk_elems(w), nc = n_chunks(d), c;
        uint8_t *co = NULL, *cn = NULL, *so = NULL, *sn = NULL;
        const orc_tensor* sd = NULL;
        if (d->numel == 0) continue;
        if (need) {   /* a tensor none of whose chunks is wanted is not read at all */
            uint64_t any = 0;
            for (c = 0; c < nc; c++) any |= need[ordinal + c];
            if (!any) { ordinal += nc; continue; }
        }
        co = (uint8_t*)malloc(d->numel * w);
        cn = (uint8_t*)malloc(d->numel * w);
        if (!co || !cn) { free(co); free(cn); rc = ORC_E_NOMEM; goto done; }
        rc = gather2(T, nT, old_shards, new_shards, shard_bytes, nS, segs, nseg, t, co, cn);
        if (rc == ORC_OK && d->route == ORC_ROUTE_BLOCK_SCALED && mode == ORC_MODE_DELTA) {
            sd = &T[d->scale_tensor];
            so = (uint8_t*)malloc(sd->numel * 4 + 1);
            sn = (uint8_t*)malloc(sd->numel * 4 + 1);
            if (!so || !sn) rc = ORC_E_NOMEM;
            else rc = gather2(T, nT, old_shards, new_shards, shard_bytes, nS, segs, nseg,
                              (uint32_t)d->scale_tensor, so, sn);
        }
        if (rc) { free(co); free(cn); free(so); free(sn); goto done; }

        for (c = 0; c < nc; c++) {
            uint64_t n_c = (d->numel - c * E < E) ? d->numel - c * E : E;
            uint64_t K[2] = {0, 0}, i;
            uint32_t k;
            if (need && !need[ordinal + c]) continue;
            for (i = 0; i < n_c; i++) {
                uint64_t g = c * E + i;
                uint32_t o = load_word(co, g, w), n = load_word(cn, g, w);
                uint32_t kind;
                if (o == n) continue; /* stored bits equal: unchanged */
                if (mode == ORC_MODE_RETRY) kind = ORC_KIND_OW;
                else if (d->route == ORC_ROUTE_AFFINE_XOR) kind = ORC_KIND_XOR;
                else if (d->route == ORC_ROUTE_OVERWRITE) kind = ORC_KIND_OW;
                else {
                    uint64_t b = g / d->scale_block;
                    kind = (load_word(so, b, 4) != load_word(sn, b, 4)) ? ORC_KIND_OW : ORC_KIND_XOR;
                }
                idx[kind][K[kind]] = (uint32_t)i;
                word[kind][K[kind]] = (kind == ORC_KIND_XOR) ? (o ^ n) : n;
                K[kind]++;
            }
            for (k = 0; k < 2; k++) {
                uint32_t hi_mode, H, layout;
                uint64_t sz;
                if (K[k] == 0) continue;
                layout = choose_layout(n_c, K[k], lists);
                sz = build_record(NULL, n_c, w, k, K[k], idx[k], word[k], layout, &hi_mode, &H);
                if ((nrec + 1) * ORC_DIRENT_BYTES <= dir_cap && poff + sz <= payload_cap) {
                    build_record(payload_out + poff, n_c, w, k, K[k], idx[k], word[k], layout, &hi_mode, &H);
                    put_dirent(dir_out + nrec * ORC_DIRENT_BYTES, t, (uint32_t)c, (uint32_t)K[k], k,
                               hi_mode, w, poff, (uint32_t)sz, H, layout);
                }
                nrec++;
                poff += sz;
            }
        }
        free(co); free(cn); free(so); free(sn);
        ordinal += nc;
    }
    *dir_bytes = nrec * ORC_DIRENT_BYTES;
    *payload_bytes = poff;
    if (nrec * ORC_DIRENT_BYTES > dir_cap || poff > payload_cap) { rc = ORC_E_CAPACITY; goto done; }
    put_header(header_out, mode, base_version, new_version, orc_fingerprint(T, nT), nrec, poff);
    rc = ORC_OK;
done:
    free(idx[0]); free(idx[1]); free(word[0]); free(word[1]);
    return rc;
}

int32_t orc_encode(const orc_tensor* T, uint32_t nT,
                   const void* const* old_shards, const void* const* new_shards,
                   const uint64_t* shard_bytes, uint32_t nS,
                   const orc_segment* segs, uint64_t nseg,
                   uint32_t mode, uint64_t base_version, uint64_t new_version,
                   uint8_t* header_out,
                   uint8_t* dir_out, uint64_t dir_cap, uint64_t* dir_bytes,
                   uint8_t* payload_out, uint64_t payload_cap, uint64_t* payload_bytes) {
    return encode_chunks(T, nT, old_shards, new_shards, shard_bytes, nS, segs, nseg, mode, base_version,
                         new_version, header_out, dir_out, dir_cap, dir_bytes, payload_out, payload_cap,
                         payload_bytes, NULL);
}

/* Partial retry: a RETRY stream over the chunks that hold at least one record
 * of the DELTA stream whose applied flag is 0 (the receiver's flags read back
 * after a failure).  The DELTA header must be a DELTA stream of this tensor
 * table (magic, format, chunk size, fingerprint); each directory entry must
 * name an existing chunk (ORC_E_FORMAT otherwise). */
int32_t orc_encode_retry_partial(const orc_tensor* T, uint32_t nT,
                                 const void* const* old_shards, const void* const* new_shards,
                                 const uint64_t* shard_bytes, uint32_t nS,
                                 const orc_segment* segs, uint64_t nseg,
                                 const uint8_t* delta_header, const uint8_t* delta_dir,
                                 const uint8_t* delta_flags,
                                 uint64_t base_version, uint64_t new_version,
                                 uint8_t* header_out,
                                 uint8_t* dir_out, uint64_t dir_cap, uint64_t* dir_bytes,
                                 uint8_t* payload_out, uint64_t payload_cap, uint64_t* payload_bytes) {
    uint64_t total = 0, n, r;
    uint64_t* first = NULL;
    uint8_t* need = NULL;
    uint32_t t;
    int32_t rc = check_tensors(T, nT);
    if (rc) return rc;
    if (get_u32(delta_header + 0) != ORC_MAGIC || get_u16(delta_header + 4) != ORC_FORMAT_VER ||
        get_u16(delta_header + 6) != ORC_MODE_DELTA || get_u32(delta_header + 8) != ORC_CHUNK_BYTES ||
        get_u64(delta_header + 32) != orc_fingerprint(T, nT))
        return ORC_E_FORMAT;
    n = get_u64(delta_header + 40);
    first = (uint64_t*)malloc((nT + 1) * sizeof(uint64_t));
    if (!first) return ORC_E_NOMEM;
    for (t = 0; t < nT; t++) {
        first[t] = total;
        total += n_chunks(&T[t]);
    }
    need = (uint8_t*)calloc(total + 1, 1);
    if (!need) { free(first); return ORC_E_NOMEM; }
    for (r = 0; r < n; r++) {
        const uint8_t* e = delta_dir + r * ORC_DIRENT_BYTES;
        uint32_t et = get_u32(e + 0), ec = get_u32(e + 4);
        if (et >= nT || ec >= n_chunks(&T[et])) { rc = ORC_E_FORMAT; goto out; }
        if (!delta_flags[r]) need[first[et] + ec] = 1;
    }
    rc = encode_chunks(T, nT, old_shards, new_shards, shard_bytes, nS, segs, nseg, ORC_MODE_RETRY,
                       base_version, new_version, header_out, dir_out, dir_cap, dir_bytes, payload_out,
                       payload_cap, payload_bytes, need);
out:
    free(first);
    free(need);
    return rc;
}

/* ------------------------------------------------------- stream parsing */

typedef struct {
    uint32_t t, c, K, kind, hi_mode, w, H, layout;
    uint64_t off, sz;
} orc_rec;

static void get_dirent(const uint8_t* p, orc_rec* r) {
    r->t = get_u32(p);
    r->c = get_u32(p + 4);
    r->K = get_u32(p + 8);
    r->kind = p[12];
    r->hi_mode = p[13];
    r->w = p[14];
    r->layout = p[15];
    r->off = get_u64(p + 16);
    r->sz = get_u32(p + 24);
    r->H = get_u32(p + 28);
}

static int bit(const uint8_t* m, uint64_t i) { return (m[i / 8] >> (i % 8)) & 1; }

/* Check every field and byte of one record against the format. */
static int32_t check_record(const orc_tensor* T, uint32_t nT, const uint8_t* dirent,
                            const uint8_t* payload, uint64_t expect_off, uint32_t stream_kind) {
    orc_rec r;
    const orc_tensor* d;
    const uint8_t* p;
    uint64_t E, n_c, i, cnt, pos, j;
    get_dirent(dirent, &r);
    if (r.layout > ORC_LAYOUT_LIST) return ORC_E_FORMAT;
    if (r.t >= nT) return ORC_E_FORMAT;
    d = &T[r.t];
    if (r.w != d->elem_bytes) return ORC_E_FORMAT;
    if ((uint64_t)r.c >= n_chunks(d)) return ORC_E_FORMAT;
    E = chunk_elems(r.w);
    n_c = (d->numel - (uint64_t)r.c * E < E) ? d->numel - (uint64_t)r.c * E : E;
    if (r.K == 0 || r.K > n_c) return ORC_E_FORMAT;
    if (r.kind > ORC_KIND_OW) return ORC_E_FORMAT;
    if (stream_kind == ORC_MODE_RETRY && r.kind != ORC_KIND_OW) return ORC_E_FORMAT;
    if (r.kind == ORC_KIND_XOR && r.w == 4) return ORC_E_FORMAT;
    if (r.off != expect_off) return ORC_E_FORMAT;
    /* mode / H consistency */
    if (r.w == 1) { if (r.hi_mode != ORC_HI_NONE || r.H != 0) return ORC_E_FORMAT; }
    else if (r.kind == ORC_KIND_OW) { if (r.hi_mode != ORC_HI_DENSE || r.H != r.K) return ORC_E_FORMAT; }
    else if (r.hi_mode == ORC_HI_NONE) { if (r.H != 0) return ORC_E_FORMAT; }
    else if (r.hi_mode == ORC_HI_SPARSE) {
        if (r.H == 0 || r.H > r.K || xor_hi_mode(r.K, r.H) != ORC_HI_SPARSE) return ORC_E_FORMAT;
    } else if (r.hi_mode == ORC_HI_DENSE) { if (r.H != r.K) return ORC_E_FORMAT; }
    else return ORC_E_FORMAT;
    if (r.sz != record_bytes(n_c, r.w, r.kind, r.K, r.hi_mode, r.H, r.layout)) return ORC_E_FORMAT;

    p = payload + r.off;
    if (r.layout == ORC_LAYOUT_LIST) {
        /* index list: K strictly ascending indices below n_c, zero padding */
        for (j = 0; j < r.K; j++) {
            uint64_t e = get_u16(p + 2 * j);
            if (e >= n_c) return ORC_E_FORMAT;
            if (j > 0 && e <= get_u16(p + 2 * (j - 1))) return ORC_E_FORMAT;
        }
        for (j = 2 * (uint64_t)r.K; j < pad16(2 * (uint64_t)r.K); j++) if (p[j]) return ORC_E_FORMAT;
    } else {
        /* bitmap: popcount K, nothing set at or beyond n_c, zero padding */
        cnt = 0;
        for (i = 0; i < pad16((n_c + 7) / 8) * 8; i++) {
            if (!bit(p, i)) continue;
            if (i >= n_c) return ORC_E_FORMAT;
            cnt++;
        }
        if (cnt != r.K) return ORC_E_FORMAT;
    }
    pos = head_bytes(n_c, r.K, r.layout);
    for (j = r.K; j < pad16(r.K); j++) if (p[pos + j]) return ORC_E_FORMAT;
    pos += pad16(r.K);
    if (r.w == 2 && r.kind == ORC_KIND_XOR && r.hi_mode == ORC_HI_SPARSE) {
        uint64_t nz = 0;
        for (j = 0; j < pad16((r.K + 7) / 8) * 8; j++) {
            if (!bit(p + pos, j)) continue;
            if (j >= r.K) return ORC_E_FORMAT;
            nz++;
        }
        if (nz != r.H) return ORC_E_FORMAT;
        pos += pad16((r.K + 7) / 8);
        for (j = 0; j < r.H; j++) if (p[pos + j] == 0) return ORC_E_FORMAT;
        for (j = r.H; j < pad16(r.H); j++) if (p[pos + j]) return ORC_E_FORMAT;
    } else if (r.w == 2 && r.kind == ORC_KIND_XOR && r.hi_mode == ORC_HI_DENSE) {
        uint64_t nz = 0;
        for (j = 0; j < r.K; j++) if (p[pos + j]) nz++;
        if (xor_hi_mode(r.K, nz) != ORC_HI_DENSE) return ORC_E_FORMAT;
        for (j = r.K; j < pad16(r.K); j++) if (p[pos + j]) return ORC_E_FORMAT;
    } else if (r.w >= 2 && r.kind == ORC_KIND_OW) {
        uint32_t b;
        for (b = 1; b < r.w; b++) {
            for (j = r.K; j < pad16(r.K); j++) if (p[pos + j]) return ORC_E_FORMAT;
            pos += pad16(r.K);
        }
    }
    return ORC_OK;
}

/* The change bitmap of a (checked) record, whatever its layout, in out
 * (pad16(n_c/8) bytes, zeroed by the caller). */
static void record_marks(const uint8_t* p, const orc_rec* r, uint64_t n_c, uint8_t* out) {
    uint64_t j;
    if (r->layout != ORC_LAYOUT_LIST) {
        memcpy(out, p, pad16((n_c + 7) / 8));
        return;
    }
    for (j = 0; j < r->K; j++) {
        uint64_t e = get_u16(p + 2 * j);
        out[e / 8] |= (uint8_t)(1u << (e % 8));
    }
}

/* Two records of one chunk may not mark elements of the same 16-byte group. */
static int32_t check_pair(const orc_tensor* T, const uint8_t* payload, const orc_rec* a, const orc_rec* b) {
    uint32_t w = a->w;
    uint64_t E = chunk_elems(w), g, i;
    uint64_t numel = T[a->t].numel;
    uint64_t n_c = (numel - (uint64_t)a->c * E < E) ? numel - (uint64_t)a->c * E : E;
    uint64_t gs = 16u / w;
    int32_t rc = ORC_OK;
    uint8_t* ma = (uint8_t*)calloc(pad16((n_c + 7) / 8) + 1, 1);
    uint8_t* mb = (uint8_t*)calloc(pad16((n_c + 7) / 8) + 1, 1);
    if (!ma || !mb) { free(ma); free(mb); return ORC_E_NOMEM; }
    record_marks(payload + a->off, a, n_c, ma);
    record_marks(payload + b->off, b, n_c, mb);
    for (g = 0; g < n_c && rc == ORC_OK; g += gs) {
        int ia = 0, ib = 0;
        for (i = g; i < g + gs && i < n_c; i++) { ia |= bit(ma, i); ib |= bit(mb, i); }
        if (ia && ib) rc = ORC_E_FORMAT;
    }
    free(ma);
    free(mb);
    return rc;
}

int32_t orc_validate(const orc_tensor* T, uint32_t nT, const uint8_t* header,
                     const uint8_t* dir, const uint8_t* payload,
                     uint64_t expected_base_version, int32_t require_kind) {
    uint64_t nrec, pbytes, r, off = 0;
    uint32_t kind;
    int32_t rc = check_tensors(T, nT);
    if (rc) return rc;
    if (get_u32(header) != ORC_MAGIC || get_u16(header + 4) != ORC_FORMAT_VER ||
        get_u32(header + 8) != ORC_CHUNK_BYTES || get_u32(header + 12) != 0 ||
        get_u64(header + 56) != 0)
        return ORC_E_FORMAT;
    kind = get_u16(header + 6);
    if (kind > ORC_MODE_RETRY) return ORC_E_FORMAT;
    if (require_kind >= 0 && kind != (uint32_t)require_kind) return ORC_E_FORMAT;
    if (get_u64(header + 32) != orc_fingerprint(T, nT)) return ORC_E_FORMAT;
    if (get_u64(header + 16) != expected_base_version) return ORC_E_VERSION;
    nrec = get_u64(header + 40);
    pbytes = get_u64(header + 48);
    for (r = 0; r < nrec; r++) {
        orc_rec cur;
        rc = check_record(T, nT, dir + r * ORC_DIRENT_BYTES, payload, off, kind);
        if (rc) return rc;
        get_dirent(dir + r * ORC_DIRENT_BYTES, &cur);
        if (cur.off + cur.sz > pbytes) return ORC_E_FORMAT;
        if (r > 0) {
            orc_rec prev;
            get_dirent(dir + (r - 1) * ORC_DIRENT_BYTES, &prev);
            /* strictly increasing (tensor, chunk, kind) */
            if (prev.t > cur.t) return ORC_E_FORMAT;
            if (prev.t == cur.t && prev.c > cur.c) return ORC_E_FORMAT;
            if (prev.t == cur.t && prev.c == cur.c) {
                if (prev.kind >= cur.kind) return ORC_E_FORMAT;
                rc = check_pair(T, payload, &prev, &cur);
                if (rc) return rc;
            }
        }
        off += cur.sz;
    }
    if (off != pbytes) return ORC_E_FORMAT;
    return ORC_OK;
}

/* ------------------------------------------------------------------ apply */

/* Decode changes [lo, hi) of one (already validated) record and apply them. */
static void apply_changes(const orc_tensor* T, void* const* canon, const uint8_t* dirent,
                          const uint8_t* payload, uint64_t lo, uint64_t hi) {
    orc_rec r;
    const orc_tensor* d;
    const uint8_t* p;
    uint64_t E, n_c, i, j = 0, rank_hi = 0;
    uint64_t lo_pos, hi_pos, pres_pos = 0;
    uint8_t* marks;
    get_dirent(dirent, &r);
    d = &T[r.t];
    E = chunk_elems(r.w);
    n_c = (d->numel - (uint64_t)r.c * E < E) ? d->numel - (uint64_t)r.c * E : E;
    p = payload + r.off;
    /* the changed elements in ascending order, from either layout */
    marks = (uint8_t*)calloc(pad16((n_c + 7) / 8) + 1, 1);
    if (!marks) return;
    record_marks(p, &r, n_c, marks);
    lo_pos = head_bytes(n_c, r.K, r.layout);
    hi_pos = lo_pos + pad16(r.K);
    if (r.hi_mode == ORC_HI_SPARSE) { pres_pos = hi_pos; hi_pos = pres_pos + pad16((r.K + 7) / 8); }
    for (i = 0; i < n_c; i++) {
        uint32_t v;
        uint64_t g;
        if (!bit(marks, i)) continue;
        /* change j sits at chunk element i */
        v = p[lo_pos + j];
        if (r.w == 2) {
            if (r.hi_mode == ORC_HI_DENSE) v |= (uint32_t)p[hi_pos + j] << 8;
            else if (r.hi_mode == ORC_HI_SPARSE && bit(p + pres_pos, j))
                v |= (uint32_t)p[hi_pos + rank_hi] << 8;
        } else if (r.w == 4) {
            uint32_t b;
            for (b = 1; b < 4; b++) v |= (uint32_t)p[hi_pos + (b - 1) * pad16(r.K) + j] << (8 * b);
        }
        if (r.hi_mode == ORC_HI_SPARSE && bit(p + pres_pos, j)) rank_hi++;
        if (j >= lo && j < hi) {
            g = (uint64_t)r.c * E + i;
            if (r.kind == ORC_KIND_XOR)
                store_word((uint8_t*)canon[r.t], g, r.w, load_word((uint8_t*)canon[r.t], g, r.w) ^ v);
            else
                store_word((uint8_t*)canon[r.t], g, r.w, v);
        }
        j++;
    }
    free(marks);
}

int32_t orc_apply(const orc_tensor* T, uint32_t nT, void* const* canon,
                  const uint8_t* header, const uint8_t* dir, const uint8_t* payload,
                  uint8_t* flags, uint64_t first, uint64_t n, uint64_t expected_base_version) {
    uint64_t r, nrec;
    int32_t rc = orc_validate(T, nT, header, dir, payload, expected_base_version, -1);
    if (rc) return rc;
    nrec = get_u64(header + 40);
    if (first > nrec || n > nrec - first) return ORC_E_INVAL;
    for (r = first; r < first + n; r++) {
        if (flags[r]) continue; /* already applied: a second XOR would undo it */
        apply_changes(T, canon, dir + r * ORC_DIRENT_BYTES, payload, 0, ~(uint64_t)0);
        flags[r] = 1;
    }
    return ORC_OK;
}

int32_t orc_apply_overwrite_retry(const orc_tensor* T, uint32_t nT, void* const* canon,
                                  const uint8_t* header, const uint8_t* dir,
                                  const uint8_t* payload, uint64_t expected_base_version) {
    uint64_t r, nrec;
    int32_t rc = orc_validate(T, nT, header, dir, payload, expected_base_version, ORC_MODE_RETRY);
    if (rc) return rc;
    nrec = get_u64(header + 40);
    for (r = 0; r < nrec; r++)
        apply_changes(T, canon, dir + r * ORC_DIRENT_BYTES, payload, 0, ~(uint64_t)0);
    return ORC_OK;
}

int32_t orc_apply_record_part(const orc_tensor* T, uint32_t nT, void* const* canon,
                              const uint8_t* dir, const uint8_t* payload,
                              uint64_t rec, uint32_t change_lo, uint32_t change_hi) {
    (void)nT;
    apply_changes(T, canon, dir + rec * ORC_DIRENT_BYTES, payload, change_lo, change_hi);
    return ORC_OK;
}

/* ------------------------------------------------ transport packing */

/* Bytes of the unsigned LEB128 form of v. */
static uint64_t leb_len(uint32_t v) {
    uint64_t n = 1;
    while (v >= 0x80u) { v >>= 7; n++; }
    return n;
}

/* Write v as unsigned LEB128 at p; returns the bytes written. */
static uint64_t leb_put(uint8_t* p, uint32_t v) {
    uint64_t n = 0;
    while (v >= 0x80u) {
        p[n++] = (uint8_t)((v & 0x7Fu) | 0x80u);
        v >>= 7;
    }
    p[n++] = (uint8_t)v;
    return n;
}

/* Bytes of the sections after the first one (low plane and upper planes),
 * which packing leaves as they are. */
static uint64_t tail_bytes(const orc_rec* r, uint64_t n_c) {
    return record_bytes(n_c, r->w, r->kind, r->K, r->hi_mode, r->H, ORC_LAYOUT_LIST) - pad16(2 * (uint64_t)r->K);
}

static uint64_t rec_n_c(const orc_tensor* T, const orc_rec* r) {
    uint64_t E = chunk_elems(r->w);
    uint64_t numel = T[r->t].numel;
    return (numel - (uint64_t)r->c * E < E) ? numel - (uint64_t)r->c * E : E;
}

int32_t orc_stream_pack(const orc_tensor* T, uint32_t nT, const uint8_t* header,
                        const uint8_t* dir, const uint8_t* payload,
                        uint8_t* header_out, uint8_t* dir_out,
                        uint8_t* payload_out, uint64_t payload_cap, uint64_t* payload_bytes) {
    uint64_t nrec, r, pos = 0, j;
    int32_t rc = orc_validate(T, nT, header, dir, payload, get_u64(header + 16), -1);
    if (rc) return rc;
    nrec = get_u64(header + 40);
    /* first the sizes, so that nothing is written when the buffer is short */
    for (r = 0; r < nrec; r++) {
        orc_rec e;
        get_dirent(dir + r * ORC_DIRENT_BYTES, &e);
        if (e.layout == ORC_LAYOUT_LIST) {
            const uint8_t* p = payload + e.off;
            uint64_t vb = 0;
            for (j = 0; j < e.K; j++) {
                uint32_t prev = j ? get_u16(p + 2 * (j - 1)) : 0;
                uint32_t gap = j ? get_u16(p + 2 * j) - prev - 1 : get_u16(p);
                vb += leb_len(gap);
            }
            if (pad16(vb) < pad16(2 * (uint64_t)e.K)) {
                pos += pad16(vb) + tail_bytes(&e, rec_n_c(T, &e));
                continue;
            }
        }
        pos += e.sz;
    }
    *payload_bytes = pos;
    if (pos > payload_cap) return ORC_E_CAPACITY;
    pos = 0;
    for (r = 0; r < nrec; r++) {
        orc_rec e;
        const uint8_t* p;
        uint8_t* d = dir_out + r * ORC_DIRENT_BYTES;
        uint64_t sz = 0;
        int packed = 0;
        get_dirent(dir + r * ORC_DIRENT_BYTES, &e);
        p = payload + e.off;
        memcpy(d, dir + r * ORC_DIRENT_BYTES, ORC_DIRENT_BYTES);
        if (e.layout == ORC_LAYOUT_LIST) {
            uint64_t vb = 0, tail = tail_bytes(&e, rec_n_c(T, &e));
            for (j = 0; j < e.K; j++) {
                uint32_t gap = j ? get_u16(p + 2 * j) - get_u16(p + 2 * (j - 1)) - 1 : get_u16(p);
                vb += leb_len(gap);
            }
            if (pad16(vb) < pad16(2 * (uint64_t)e.K)) {
                uint64_t q = 0;
                memset(payload_out + pos, 0, pad16(vb));
                for (j = 0; j < e.K; j++) {
                    uint32_t gap = j ? get_u16(p + 2 * j) - get_u16(p + 2 * (j - 1)) - 1 : get_u16(p);
                    q += leb_put(payload_out + pos + q, gap);
                }
                memcpy(payload_out + pos + pad16(vb), p + pad16(2 * (uint64_t)e.K), tail);
                sz = pad16(vb) + tail;
                d[15] = ORC_LAYOUT_GAPS;
                packed = 1;
            }
        }
        if (!packed) {
            memcpy(payload_out + pos, p, e.sz);
            sz = e.sz;
        }
        put_u64(d + 16, pos);
        put_u32(d + 24, (uint32_t)sz);
        pos += sz;
    }
    memcpy(header_out, header, ORC_HEADER_BYTES);
    put_u32(header_out, ORC_MAGIC_PACKED);
    put_u64(header_out + 48, pos);
    return ORC_OK;
}

int32_t orc_stream_unpack(const orc_tensor* T, uint32_t nT, const uint8_t* header,
                          const uint8_t* dir, const uint8_t* payload,
                          uint8_t* header_out, uint8_t* dir_out,
                          uint8_t* payload_out, uint64_t payload_cap, uint64_t* payload_bytes) {
    uint64_t nrec, pbytes, r, pos = 0, off = 0;
    int32_t rc = check_tensors(T, nT);
    if (rc) return rc;
    if (get_u32(header) != ORC_MAGIC_PACKED || get_u16(header + 4) != ORC_FORMAT_VER ||
        get_u32(header + 8) != ORC_CHUNK_BYTES || get_u32(header + 12) != 0 || get_u64(header + 56) != 0 ||
        get_u16(header + 6) > ORC_MODE_RETRY || get_u64(header + 32) != orc_fingerprint(T, nT))
        return ORC_E_FORMAT;
    nrec = get_u64(header + 40);
    pbytes = get_u64(header + 48);
    /* sizes first: every entry's own fields give its unpacked size */
    for (r = 0; r < nrec; r++) {
        orc_rec e;
        get_dirent(dir + r * ORC_DIRENT_BYTES, &e);
        if (e.t >= nT || e.w != T[e.t].elem_bytes || (uint64_t)e.c >= n_chunks(&T[e.t])) return ORC_E_FORMAT;
        if (e.off != off || e.off + e.sz > pbytes) return ORC_E_FORMAT;
        off += e.sz;
        if (e.layout == ORC_LAYOUT_GAPS)
            pos += record_bytes(rec_n_c(T, &e), e.w, e.kind, e.K, e.hi_mode, e.H, ORC_LAYOUT_LIST);
        else
            pos += e.sz;
    }
    if (off != pbytes) return ORC_E_FORMAT;
    *payload_bytes = pos;
    if (pos > payload_cap) return ORC_E_CAPACITY;
    pos = 0;
    for (r = 0; r < nrec; r++) {
        orc_rec e;
        const uint8_t* p;
        uint8_t* d = dir_out + r * ORC_DIRENT_BYTES;
        uint64_t sz;
        get_dirent(dir + r * ORC_DIRENT_BYTES, &e);
        p = payload + e.off;
        memcpy(d, dir + r * ORC_DIRENT_BYTES, ORC_DIRENT_BYTES);
        if (e.layout == ORC_LAYOUT_GAPS) {
            uint64_t n_c = rec_n_c(T, &e), tail, sec, q = 0, j;
            uint32_t prev = 0;
            if (e.K == 0 || e.K > n_c) return ORC_E_FORMAT;
            tail = tail_bytes(&e, n_c);
            if (e.sz < tail) return ORC_E_FORMAT;
            sec = e.sz - tail;             /* the padded gap section */
            if (sec % 16 || sec >= pad16(2 * (uint64_t)e.K)) return ORC_E_FORMAT;
            sz = pad16(2 * (uint64_t)e.K) + tail;
            memset(payload_out + pos, 0, pad16(2 * (uint64_t)e.K));
            for (j = 0; j < e.K; j++) {
                uint32_t v = 0, shift = 0, idx;
                uint64_t start = q;
                for (;;) {
                    uint8_t b;
                    if (q >= sec || shift > 14) return ORC_E_FORMAT;   /* cut off, or past 3 bytes */
                    b = p[q++];
                    v |= (uint32_t)(b & 0x7Fu) << shift;
                    shift += 7;
                    if (!(b & 0x80u)) {
                        if (q - start > 1 && b == 0) return ORC_E_FORMAT;   /* not minimal */
                        break;
                    }
                }
                if (v > 0xFFFFu) return ORC_E_FORMAT;
                idx = j ? prev + 1 + v : v;
                if (idx >= n_c) return ORC_E_FORMAT;
                put_u16(payload_out + pos + 2 * j, (uint16_t)idx);
                prev = idx;
            }
            for (; q < sec; q++)
                if (p[q]) return ORC_E_FORMAT;
            memcpy(payload_out + pos + pad16(2 * (uint64_t)e.K), p + sec, tail);
            d[15] = ORC_LAYOUT_LIST;
        } else {
            memcpy(payload_out + pos, p, e.sz);
            sz = e.sz;
        }
        put_u64(d + 16, pos);
        put_u32(d + 24, (uint32_t)sz);
        pos += sz;
    }
    memcpy(header_out, header, ORC_HEADER_BYTES);
    put_u32(header_out, ORC_MAGIC);
    put_u64(header_out + 48, pos);
    return orc_validate(T, nT, header_out, dir_out, payload_out, get_u64(header_out + 16), -1);
}
