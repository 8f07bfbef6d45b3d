"""Planted mistakes in the oracle must be caught by the pins.

Each mutant is a copy of oracle.c with one plausible mistake (a dropped term,
a wrong sign or index, a transposed operand, a wrong tie rule ...), compiled
with gcc into a temporary directory. The pin suite must fail on every one of
them; otherwise the pins would not be able to tell a correct oracle from a
subtly wrong one.
"""
import os

import pytest

from oracle import SRC_PATH, Oracle, build, load
from pins import ALL_PINS

MUTANTS = {
    "markov_dropped": ("zp[v] = (float)(z_row[v] + m[v]);", "zp[v] = (float)(z_row[v]);"),
    "markov_sign": ("zp[v] = (float)(z_row[v] + m[v]);", "zp[v] = (float)(z_row[v] - m[v]);"),
    "markov_w1_w2_swapped": ("const uint16_t* u = w1 + (long)prev * r;",
                             "const uint16_t* u = w2 + (long)prev * r; w2 = w1;"),
    "prev_never_updated": ("prev = tokens[j];", "prev = anchor;"),
    "prev0_not_anchor": ("int prev = anchor;", "int prev = 0;"),
    "argmax_last_tie": ("if (zp[v] > zp[best])\n            best = v;\n    return best;",
                        "if (zp[v] >= zp[best])\n            best = v;\n    return best;"),
    "bias_dropped": ("s += (double)bias[v];", "s += 0.0;"),
    "bonus_slot_read": ("load_hidden_row(hidden, hidden_is_f32, (long)b * L + i_first_pred + j, H, x + (size_t)j * H);",
                        "load_hidden_row(hidden, hidden_is_f32, (long)b * L + j, H, x + (size_t)j * H);"),
    "lm_head_transposed": ("s += xj[h] * bf16_value(w[h]);",
                           "s += xj[h] * bf16_value(lm_head[(long)h * V + v]);"),
    "truncate_le": ("if (conf[j] < p_min)", "if (conf[j] <= p_min)"),
    "sigmoid_sign": ("return (float)(1.0 / (1.0 + exp(-c)));", "return (float)(1.0 / (1.0 + exp(c)));"),
    "rne_ties_down": ("return (lo & 1u) ? hi : lo;", "return lo;"),
    "topk_no_exclusion": ("taken = 1;", "taken = 0;"),
    "topk_last_tie": ("if (best < 0 || zp[v] > zp[best])", "if (best < 0 || zp[v] >= zp[best])"),
    "conf_wrong_slot": ("load_hidden_row(hidden, hidden_is_f32, (long)b * L + i_first_pred + j, H, x);",
                        "load_hidden_row(hidden, hidden_is_f32, (long)b * L + j, H, x);"),
    "truncate_short": ("            return j;\n    return n_pred;", "            return j;\n    return n_pred - 1;"),
    "markov_rank_short": ("for (int k = 0; k < r; ++k)", "for (int k = 1; k < r; ++k)"),
    "d2t_prev_is_draft_id": ("prev_tok = (int)d2t[best];", "prev_tok = best;"),
    "d2t_prev0_not_anchor": ("int prev_tok = anchor;", "int prev_tok = 0;"),
    "d2t_token_unmapped": ("tokens[j] = (int32_t)d2t[best];", "tokens[j] = best;"),
    "d2t_candidates_unmapped": ("cand[(size_t)j * top_k + t] = (int32_t)d2t[idx[t]];",
                                "cand[(size_t)j * top_k + t] = idx[t];"),
    "d2t_markov_dropped": ("zp[i] = (float)(zj[i] + m);", "zp[i] = (float)(zj[i]);"),
    "d2t_w1_by_draft_row": ("const uint16_t* u = r > 0 ? w1 + (long)prev_tok * r : NULL;",
                            "const uint16_t* u = r > 0 ? w1 + (long)(prev_tok % D) * r : NULL;"),
    "verify_no_length_cap": ("        while (m < len) {", "        while (m < n_pred) {"),
    "verify_lattice_first_only": ("            for (int i = 0; i < width; ++i)\n                if (c[i] == t)",
                                  "            for (int i = 0; i < 1; ++i)\n                if (c[i] == t)"),
    "verify_counts_all_matches": ("            if (!found)\n                break;\n            ++m;",
                                  "            if (!found) {\n                ++m;\n                continue;\n            }\n            ++m;"),
    "verify_total_unclamped": ("        totals[1] += len;", "        totals[1] += lengths[b];"),
    "gated_chain_ignores_cut": ("st = oracle_block_chain(zz, w1, w2, V, r, anchors[b], len, kb, tokens, c, cv);",
                                "st = oracle_block_chain(zz, w1, w2, V, r, anchors[b], len, kb, tokens, c, cv); tokens[len - 1] = 0;"),
    "gated_keeps_all_candidates": ("                for (int t = 0; t < kb; ++t) {\n                    cand[(size_t)j * top_k + t]",
                                   "                for (int t = 0; t < kb - 1; ++t) {\n                    cand[(size_t)j * top_k + t]"),
    "gated_no_fill": ("            cand_val[(size_t)j * top_k + t] = -INFINITY;", "            cand_val[(size_t)j * top_k + t] = 0.0f;"),
    "q4_low_nibble_is_high": ("w[i * Q4_BLOCK + j] = d * (double)((int)(qs[j] & 0x0f) - 8);",
                              "w[i * Q4_BLOCK + j] = d * (double)((int)(qs[j] >> 4) - 8);"),
    "q4_offset_7": ("w[i * Q4_BLOCK + j + 16] = d * (double)((int)(qs[j] >> 4) - 8);",
                    "w[i * Q4_BLOCK + j + 16] = d * (double)((int)(qs[j] >> 4) - 7);"),
    "q4_interleaved_nibbles": (
        "w[i * Q4_BLOCK + j] = d * (double)((int)(qs[j] & 0x0f) - 8);\n"
        "            w[i * Q4_BLOCK + j + 16] = d * (double)((int)(qs[j] >> 4) - 8);",
        "w[i * Q4_BLOCK + 2 * j] = d * (double)((int)(qs[j] & 0x0f) - 8);\n"
        "            w[i * Q4_BLOCK + 2 * j + 1] = d * (double)((int)(qs[j] >> 4) - 8);"),
    "q4_scale_big_endian": ("f16_value((uint16_t)(blk[0] | (blk[1] << 8)))",
                            "f16_value((uint16_t)(blk[1] | (blk[0] << 8)))"),
    "q4_scale_read_as_bf16": ("const double d = f16_value(", "const double d = bf16_value("),
    "q4_block_stride_16": ("const uint8_t* blk = row + (long)i * Q4_BLOCK_BYTES;",
                           "const uint8_t* blk = row + (long)i * 16;"),
    "q4_row_stride_unpadded": ("const uint8_t* row = q4 + v * (long)nb * Q4_BLOCK_BYTES;",
                               "const uint8_t* row = q4 + v * (long)nb * 16;"),
    "f16_subnormal_as_normal": ("v = ldexp((double)f, -24);", "v = ldexp((double)(1024 + f), -25);"),
    "f16_exponent_bias": ("v = ldexp((double)(1024 + f), e - 25);", "v = ldexp((double)(1024 + f), e - 24);"),
    "f16_sign_dropped": ("return (bits & 0x8000u) ? -v : v;", "return v;"),
    "q4_bias_dropped": ("s = s + (double)bias[v];", "s = s + 0.0;"),
    "q4_bonus_slot_read": ("const long first_row = (long)b * L + i_first_pred;",
                           "const long first_row = (long)b * L;"),
    "q4_last_row_skipped": ("for (long v = 0; v < V; ++v) {\n            if (!w) {",
                            "for (long v = 0; v < V - 1; ++v) {\n            if (!w) {"),
    "hidden_f32_truncated": ("x[h] = bf16_value(oracle_bf16_round(p[h]));",
                             "x[h] = bf16_value((uint16_t)(*(const uint32_t*)&p[h] >> 16));"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC_PATH) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = tmp_path / "oracle_mutant.c"
    src.write_text(source.replace(old, new))
    lib = load(build(str(src), str(tmp_path / "liboracle_mutant.so")))
    orc = Oracle(lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
        except ValueError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
