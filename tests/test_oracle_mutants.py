"""Planted mistakes in a copy of the oracle must each fail at least one pin.

Each mutant is a plausible slip (wrong bit order, float-style comparison,
wrong word, tie-break, byte plane, transposed strides, chunk size, missing
dedup, inverted routing, missing padding, partial retry ignoring the flags or
marking the wrong chunk, index lists off by one or never chosen, the same-group
check between a chunk's two records skipped, a header field left unwritten,
tensor-table refusals dropped, gap varints off by one or never ending, packing
on a size tie, longer varints accepted); the copy is compiled in a temp
directory and loaded beside the real oracle.  Nothing here touches a GPU.
"""
import os
import shutil

import pytest

from oracle import oracle as O
from tests import pins

SRC = os.path.join(os.path.dirname(O.__file__), "dcr_oracle.c")

MUTANTS = {
    "bitmap_msb_first": ("out[idx[j] / 8] |= (uint8_t)(1u << (idx[j] % 8));",
                         "out[idx[j] / 8] |= (uint8_t)(0x80u >> (idx[j] % 8));"),
    "float_style_compare": ("if (o == n) continue; /* stored bits equal: unchanged */",
                            "if (o == n || (w == 2 && ((o | n) & 0x7FFF) == 0)) continue;"),
    "xor_word_is_new": ("word[kind][K[kind]] = (kind == ORC_KIND_XOR) ? (o ^ n) : n;",
                        "word[kind][K[kind]] = n;"),
    "hi_mode_tie_sparse": ("if (pad16((K + 7) / 8) + pad16(h) < pad16(K)) return ORC_HI_SPARSE;",
                           "if (pad16((K + 7) / 8) + pad16(h) <= pad16(K)) return ORC_HI_SPARSE;"),
    "lo_plane_wrong_byte": ("for (j = 0; j < K; j++) out[pos + j] = (uint8_t)(word[j] & 0xFF);",
                            "for (j = 0; j < K; j++) out[pos + j] = (uint8_t)(word[j] >> 8);"),
    "projection_strides_swapped": ("c += (int64_t)x[k] * g->canon_stride[k];",
                                   "c += (int64_t)x[k] * g->shard_stride[k];"),
    "chunk_elems_fixed": ("static uint64_t chunk_elems(uint32_t w) { return ORC_CHUNK_BYTES / w; }",
                          "static uint64_t chunk_elems(uint32_t w) { (void)w; return ORC_CHUNK_BYTES / 2; }"),
    "no_dedup": ("if (flags[r]) continue; /* already applied: a second XOR would undo it */",
                 "(void)0;"),
    "block_route_inverted": ("kind = (load_word(so, b, 4) != load_word(sn, b, 4)) ? ORC_KIND_OW : ORC_KIND_XOR;",
                             "kind = (load_word(so, b, 4) != load_word(sn, b, 4)) ? ORC_KIND_XOR : ORC_KIND_OW;"),
    "no_padding": ("static uint64_t pad16(uint64_t x) { return (x + 15u) & ~(uint64_t)15u; }",
                   "static uint64_t pad16(uint64_t x) { return x; }"),
    "sparse_rank_not_advanced": ("if (r.hi_mode == ORC_HI_SPARSE && bit(p + pres_pos, j)) rank_hi++;",
                                 "(void)0;"),
    "shard_offset_dropped": ("int64_t c = (int64_t)g->canon_off, e = (int64_t)g->shard_off;",
                             "int64_t c = (int64_t)g->canon_off, e = 0;"),
    "partial_retry_ignores_flags": ("if (!delta_flags[r]) need[first[et] + ec] = 1;",
                                    "need[first[et] + ec] = 1;"),
    "partial_retry_wrong_chunk": ("if (!delta_flags[r]) need[first[et] + ec] = 1;",
                                  "if (!delta_flags[r]) need[first[et]] = 1;"),
    "list_index_off_by_one": ("for (j = 0; j < K; j++) put_u16(out + 2 * j, (uint16_t)idx[j]);",
                              "for (j = 0; j < K; j++) put_u16(out + 2 * j, (uint16_t)(idx[j] + 1));"),
    "check_pair_skipped": ("rc = check_pair(T, payload, &prev, &cur);",
                           "rc = ORC_OK;"),
    "header_new_version_dropped": ("put_u64(p + 24, new_v);", "(void)new_v;"),
    "xor_on_w4_allowed": ("if (d->route != ORC_ROUTE_OVERWRITE && w == 4) return ORC_E_INVAL;", "(void)0;"),
    "scale_length_unchecked": ("if (s->numel != (d->numel + d->scale_block - 1) / d->scale_block) return ORC_E_INVAL;",
                               "(void)s;"),
    "gap_written_without_minus_one": ("q += leb_put(payload_out + pos + q, gap);",
                                      "q += leb_put(payload_out + pos + q, gap + (j ? 1u : 0u));"),
    "leb128_continuation_on_last": ("p[n++] = (uint8_t)v;", "p[n++] = (uint8_t)(v | 0x80u);"),
    "pack_on_a_tie": ("if (pad16(vb) < pad16(2 * (uint64_t)e.K)) {\n                uint64_t q = 0;",
                      "if (pad16(vb) <= pad16(2 * (uint64_t)e.K)) {\n                uint64_t q = 0;"),
    "unpack_accepts_longer_varints": ("if (q - start > 1 && b == 0) return ORC_E_FORMAT;   /* not minimal */",
                                      "(void)start;"),
    "list_layout_never": ("return (lists && pad16(2 * K) < pad16((n_c + 7) / 8)) ? ORC_LAYOUT_LIST : ORC_LAYOUT_BITMAP;",
                          "(void)lists; (void)K; (void)n_c; return ORC_LAYOUT_BITMAP;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, name
    d = tmp_path / "src"
    d.mkdir()
    shutil.copy(os.path.join(os.path.dirname(SRC), "dcr_oracle.h"), d / "dcr_oracle.h")
    (d / "dcr_oracle.c").write_text(src.replace(before, after))
    lib = O.build(force=True, src_dir=str(d), out_path=str(tmp_path / f"lib_{name}.so"),
                  extra_flags=("-Wno-unused-parameter", "-Wno-unused-variable"))
    mut = O.Oracle(lib)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(mut)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            failed.append((pin.__name__, type(e).__name__))
            break
    assert failed, f"mutant {name} passed every pin"
