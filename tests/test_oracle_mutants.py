"""Plant plausible mistakes in copies of the oracle and check the pins catch each one.

Every mutant is a one-line edit of oracle.c (a dropped term, a wrong sign, a
transposed index, an off-by-one bound), compiled on the CPU into a temporary
library and run through the same pin functions in a child process (a broken
index may crash it, which also counts as caught).
"""
import os
import subprocess
import sys

import pytest

from oracle.build import SOURCE, build_oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

MUTANTS = {
    "paged_offset_sign": ("if (logical >= bound) continue;            /* no block owned there: pad id */\n            int64_t physical = block_table[(int64_t)r * table_stride + logical];\n            if (physical < 0) { flags |= ORC_FLAG_BAD_BLOCK; continue; }\n            slot_mapping[t] = physical * block_size + offset;",
                          "if (logical >= bound) continue;            /* no block owned there: pad id */\n            int64_t physical = block_table[(int64_t)r * table_stride + logical];\n            if (physical < 0) { flags |= ORC_FLAG_BAD_BLOCK; continue; }\n            slot_mapping[t] = physical * block_size - offset;"),
    "ranges_offset_dropped": ("if (physical < 0) flags |= ORC_FLAG_BAD_BLOCK;\n                    else slot_mapping[t] = physical * block_size + offset;\n                    break;\n                }\n            }\n        }\n    }\n    if (flags_out) *flags_out |= flags;\n    return ORC_OK;\n}\n\n/*\n * Context-parallel",
                              "if (physical < 0) flags |= ORC_FLAG_BAD_BLOCK;\n                    else slot_mapping[t] = physical * block_size;\n                    break;\n                }\n            }\n        }\n    }\n    if (flags_out) *flags_out |= flags;\n    return ORC_OK;\n}\n\n/*\n * Context-parallel"),
    "offset_is_quotient": ("int64_t offset = p % block_size;\n            if (logical >= bound)",
                           "int64_t offset = p / block_size;\n            if (logical >= bound)"),
    "bound_off_by_one": ("if (logical >= bound) continue;            /* no block owned there: pad id */",
                         "if (logical > bound) continue;             /* no block owned there: pad id */"),
    "table_transposed": ("/* no block owned there: pad id */\n            int64_t physical = block_table[(int64_t)r * table_stride + logical];",
                         "/* no block owned there: pad id */\n            int64_t physical = block_table[(int64_t)logical * table_stride + r];"),
    "range_sign": ("int64_t offset = p % block_size;\n            for (int64_t i = 0; i < n; ++i) {\n                int64_t k = (int64_t)r * range_stride + i;\n                int64_t cum = range_cum[k], len = range_len[k];\n                if (cum <= logical && logical < cum + len) {\n                    int64_t physical = (int64_t)range_start[k] + (logical - cum);",
                   "int64_t offset = p % block_size;\n            for (int64_t i = 0; i < n; ++i) {\n                int64_t k = (int64_t)r * range_stride + i;\n                int64_t cum = range_cum[k], len = range_len[k];\n                if (cum <= logical && logical < cum + len) {\n                    int64_t physical = (int64_t)range_start[k] + (cum - logical);"),
    "range_end_inclusive": ("int64_t offset = p % block_size;\n            for (int64_t i = 0; i < n; ++i) {\n                int64_t k = (int64_t)r * range_stride + i;\n                int64_t cum = range_cum[k], len = range_len[k];\n                if (cum <= logical && logical < cum + len) {",
                            "int64_t offset = p % block_size;\n            for (int64_t i = 0; i < n; ++i) {\n                int64_t k = (int64_t)r * range_stride + i;\n                int64_t cum = range_cum[k], len = range_len[k];\n                if (cum <= logical && logical <= cum + len) {"),
    "range_drops_cum": ("int64_t offset = p % block_size;\n            for (int64_t i = 0; i < n; ++i) {\n                int64_t k = (int64_t)r * range_stride + i;\n                int64_t cum = range_cum[k], len = range_len[k];\n                if (cum <= logical && logical < cum + len) {\n                    int64_t physical = (int64_t)range_start[k] + (logical - cum);",
                        "int64_t offset = p % block_size;\n            for (int64_t i = 0; i < n; ++i) {\n                int64_t k = (int64_t)r * range_stride + i;\n                int64_t cum = range_cum[k], len = range_len[k];\n                if (cum <= logical && logical < cum + len) {\n                    int64_t physical = (int64_t)range_start[k] + logical;"),
    "expansion_drops_factor": ("if (expandable(id, k)) v = id * k + j;",
                               "if (expandable(id, k)) v = id + j;"),
    "expansion_tail_not_null": ("for (int64_t c = 0; c < out_stride; ++c) out[(int64_t)r * out_stride + c] = 0;",
                                "for (int64_t c = 0; c < out_stride; ++c) out[(int64_t)r * out_stride + c] = 1;"),
    "fill_drops_factor": ("if (expandable(b, k)) row[length] = (int32_t)(b * k + j);",
                          "if (expandable(b, k)) row[length] = (int32_t)(b + j);"),
    "fill_drops_sub_block": ("if (expandable(b, k)) row[length] = (int32_t)(b * k + j);",
                             "if (expandable(b, k)) row[length] = (int32_t)(b * k);"),
    "fill_run_end_inclusive": ("for (int64_t b = start[d]; b < (int64_t)start[d] + len[d]; ++b) {",
                               "for (int64_t b = start[d]; b <= (int64_t)start[d] + len[d]; ++b) {"),
    "fill_tail_not_null": ("for (int64_t q = 0; q < out_stride; ++q) row[q] = 0;",
                           "for (int64_t q = 0; q < out_stride; ++q) row[q] = 1;"),
    "fill_count_unclamped": ("counts_out[r] = (int32_t)(full < out_stride ? full : out_stride);",
                             "counts_out[r] = (int32_t)full;"),
    "cp_owner_uses_remainder": ("if ((p / I) % W != cp_rank) continue;      /* another rank's position */\n            int64_t bound",
                                "if ((p % I) % W != cp_rank) continue;      /* another rank's position */\n            int64_t bound"),
    "cp_offset_drops_chunk": ("int64_t offset = (o / (I * W)) * I + o % I;\n            if (logical >= bound) continue;",
                              "int64_t offset = o % I;\n            if (logical >= bound) continue;"),
    "cp_block_not_widened": ("int64_t logical = p / span;\n            int64_t o = p % span;\n            int64_t offset = (o / (I * W)) * I + o % I;\n            if (logical >= bound)",
                             "int64_t logical = p / block_size;\n            int64_t o = p % span;\n            int64_t offset = (o / (I * W)) * I + o % I;\n            if (logical >= bound)"),
    "cp_ranges_offset_global": ("int64_t offset = (o / (I * W)) * I + o % I;\n            for (int64_t i = 0; i < n; ++i) {",
                                "int64_t offset = o;\n            for (int64_t i = 0; i < n; ++i) {"),
    "expansion_counts_unscaled": ("if (counts_out) counts_out[r] = (int32_t)(count * k);",
                                  "if (counts_out) counts_out[r] = (int32_t)count;"),
    "attention_lse_without_max": ("lse_out[(int64_t)i * num_q_heads + h] = smax + log(denom);",
                                  "lse_out[(int64_t)i * num_q_heads + h] = log(denom);"),
    "attention_drops_scale": ("    return sc * scale;\n}", "    return sc;\n}"),
    "attention_heads_interleaved": ("            int64_t g = h / group;", "            int64_t g = h % num_kv_heads;"),
    "attention_no_max_shift": ("denom += exp(attention_score(qh, kr, head_dim, scale) - smax);",
                               "denom += exp(attention_score(qh, kr, head_dim, scale));"),
    "attention_unnormalized": ("double w = exp(attention_score(qh, kr, head_dim, scale) - smax) / denom;",
                               "double w = exp(attention_score(qh, kr, head_dim, scale) - smax);"),
    "attention_keys_as_values": ("for (int32_t d = 0; d < head_dim; ++d) o[d] += w * bf16_value(vr[d]);",
                                 "for (int32_t d = 0; d < head_dim; ++d) o[d] += w * bf16_value(kr[d]);"),
    "coord_swaps_B_T": ("return (layer * num_blocks + block) * block_size + token;",
                        "return (layer * block_size + block) * num_blocks + token;"),
    "kv_drops_layer_term": ("int64_t src = layer * kv_layer_stride + t * kv_token_stride;",
                            "int64_t src = t * kv_token_stride;"),
    "tail_not_padded": ("/* no token rows: nothing is read */\n    for (int64_t t = 0; t < max_num_tokens; ++t) slot_mapping[t] = ORC_PAD_ID;",
                        "/* no token rows: nothing is read */\n    for (int64_t t = 0; t < max_num_tokens; ++t) slot_mapping[t] = 0;"),
    "request_end_inclusive": ("for (int64_t t = qsl[r]; t < qsl[r + 1] && t < num_tokens; ++t) {\n            int64_t p = positions[t];\n            if (p < 0) continue;                       /* pad id */",
                              "for (int64_t t = qsl[r]; t <= qsl[r + 1] && t < num_tokens; ++t) {\n            int64_t p = positions[t];\n            if (p < 0) continue;                       /* pad id */"),
    "negative_position_kept": ("if (p < 0) continue;                       /* pad id */",
                               "if (p < -1) continue;                      /* pad id */"),
    "pad_rows_written": ("if (s < 0) continue;                         /* padded token: no write */",
                         "if (s < 0) s = 0;                            /* padded token: no write */"),
}

CHILD = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle, oracle_pins as P
from workloads import small_cases
orc = oracle.Oracle({lib!r})
small = [w for w in small_cases() if w.name in ("tiny_prefill", "small_bs8", "small_layers",
         "small_out_of_range", "small_dummy", "small_row256", "small_long_r4")]
P.all_pins(orc, small)
print("ALL PINS PASSED")
"""


def test_unmutated_copy_passes(tmp_path):
    lib = str(tmp_path / "liboracle_copy.so")
    build_oracle(output=lib)
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, tests=HERE, lib=lib)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "ALL PINS PASSED" in r.stdout, r.stderr[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SOURCE).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = str(tmp_path / "liboracle_mut.so")
    build_oracle(output=lib, source=str(mutated), extra_flags=("-Wno-error",))
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, tests=HERE, lib=lib)],
                       capture_output=True, text=True, timeout=300)
    assert "ALL PINS PASSED" not in r.stdout, f"mutant {name} survived every pin"
