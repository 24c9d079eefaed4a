"""The pins catch plausible mistakes: each mutant below is a copy of the oracle with one
planted error (built on the CPU into a temporary directory); at least one pin must fail on it.
None of the mutants reads or writes out of bounds."""
import os

import pytest

from oracle import build as obuild
from oracle.ref import Oracle
from tests import oracle_pins

SRC = open(obuild.SRC).read()

MUTANTS = {
    "pairwise_mean": ("float s = k0 + k1;\n    s = s + k2;\n    s = s + k3;",
                      "float s = (k0 + k1) + (k2 + k3);"),
    "reversed_mean": ("float s = k0 + k1;\n    s = s + k2;\n    s = s + k3;",
                      "float s = k3 + k2;\n    s = s + k1;\n    s = s + k0;"),
    "mean_not_cast": ("m[d] = widen(mT, dt);", "m[d] = mean;"),
    "gamma_prefolded": ("float w1 = 1.0f + widen(w[d], dt);", "float w1 = widen(w[d], dt);"),
    "rope_sign_low": ("o[i] = a0 - b0;", "o[i] = a0 + b0;"),
    "rope_sign_high": ("o[i + HALF_ROPE] = a1 + b1;", "o[i + HALF_ROPE] = a1 - b1;"),
    "cos_sin_swapped": ("float c = cs[i], s = cs[HALF_ROPE + i];",
                        "float s = cs[i], c = cs[HALF_ROPE + i];"),
    "rope_on_wrong_half": ("for (int d = 2 * HALF_ROPE; d < DIM; ++d) o[d] = y[d];",
                           "for (int d = 2 * HALF_ROPE; d < DIM; ++d) o[d] = y[d] * cs[0];"),
    "mean_over_64": ("float meanSq = sumSq / 128.0f;", "float meanSq = sumSq / 64.0f;"),
    "eps_dropped": ("float v = meanSq + eps;", "float v = meanSq;"),
    "rope_at_g": ("cosSin + 4 * g * CS_W", "cosSin + g * CS_W"),
    "padding_off_by_one": ("if (t >= L) {", "if (t > L) {"),
    "no_pastlen_rule": ("if (!(t0 >= p)) return 0;", "(void)p;"),
    "row_map_ignores_past": ("(4 * g + j - p)) * ROW + KCOL", "(4 * g + j - p + (p > 0))) * ROW + KCOL"),
    "tail_start_wrong": ("int64_t t0 = c - c % 4;", "int64_t t0 = c - 4;"),
    "v_tail_on_k_plane": ("int64_t off = pool_tail_offset(pool, b, 1, 4 * g);\n      if (off >= 0) memcpy(base",
                          "int64_t off = pool_tail_offset(pool, b, 0, 4 * g);\n      if (off >= 0) memcpy(base"),
    "headsize_dropped": ("+ 0 * p->poolHeadDim + p->headSize;", "+ 0 * p->poolHeadDim + 0;"),
    "page_row_wrong": ("int64_t row = pos % PAGE;", "int64_t row = (pos + 1) % PAGE;"),
    "bf16_truncates": ("if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;",
                       "(void)rest;"),
    "bf16_ties_away": ("(rest == 0x8000u && (keep & 1u))", "(rest == 0x8000u)"),
    "f16_no_subnormal": ("int drop = (e >= -14) ? 13 : 13 + (-14 - e);",
                         "if (e < -14) return sign;\n  int drop = 13;"),
    "decode_rope_position": ("norm_rope(x, wQ, cosSin + t * CS_W, eps, dt, qb",
                             "norm_rope(x, wQ, cosSin + (t + 1) * CS_W, eps, dt, qb"),
    "decode_first_block_skipped": ("for (int64_t g = p / 4;", "for (int64_t g = (p + 3) / 4;"),
    "decode_tails_of_completed_blocks": ("int64_t t0 = c - c % 4;\n    if (t0 < p) t0 = p;\n    for",
                                         "int64_t t0 = p;\n    for"),
    "decode_past_keys_wrong_plane": ("int64_t off = pool_tail_offset(pool, b, 0, t);\n          if (off < 0) ok = 0;",
                                     "int64_t off = pool_tail_offset(pool, b, 1, t);\n          if (off < 0) ok = 0;"),
    "score_relu_after_sum": ("float relu = dot > 0.0f ? dot : 0.0f;\n    sum = sum + relu;\n  }\n  return score_scale() * sum;",
                             "sum = sum + dot;\n  }\n  return score_scale() * (sum > 0.0f ? sum : 0.0f);"),
    "score_scale_before_sum": ("sum = sum + relu;\n  }\n  return score_scale() * sum;",
                               "sum = sum + score_scale() * relu;\n  }\n  return sum;"),
    "score_nvis_off_by_one": ("int64_t nVis = (t + 1) / 4;", "int64_t nVis = (t + 4) / 4;"),
    "score_padding_rule": ("if (c <= 0 || t >= c) {", "if (c <= 0 || t > c) {"),
    "score_decode_plane": ("int64_t off = pool_tail_offset(pool, b, 1, 4 * g);\n      logits",
                           "int64_t off = pool_tail_offset(pool, b, 0, 4 * g);\n      logits"),
    "expand_no_tail": ("  for (int64_t j = 0; j < tail; ++j) out[n++] = (int32_t)(4 * nVis + j);\n  while",
                       "  (void)tail;\n  while"),
    "topk_511": ("enum { TOPK = 512, INDEX_WIDTH = 2051 };", "enum { TOPK = 511, INDEX_WIDTH = 2051 };"),
    "ties_descending_id": ("return a->id < b->id ? -1 : (a->id > b->id);",
                           "return a->id > b->id ? -1 : (a->id < b->id);"),
    "orderable_negatives_uncomplemented": ("return (b & 0x80000000u) ? ~b : (b | 0x80000000u);",
                                           "return (b & 0x80000000u) ? (b & 0x7fffffffu) : (b | 0x80000000u);"),
    "decode_emits_sorted_order": ("      for (int64_t g = 0; g < nVis; ++g)\n        if (pick[g]) sel[n++] = (int32_t)g;",
                                  "      for (int64_t i = 0; i < kSel; ++i) sel[n++] = kv[i].id;"),
    "expand_padded_rule": ("    if (ctx[b] <= 0 || t >= ctx[b]) {\n      for (int k = 0; k < INDEX_WIDTH; ++k) out[k] = -1;\n      continue;\n    }\n    int64_t nVis = (t + 1) / 4;\n    expand_row(out, sortedIds",
                           "    if (ctx[b] <= 0 || t > ctx[b]) {\n      for (int k = 0; k < INDEX_WIDTH; ++k) out[k] = -1;\n      continue;\n    }\n    int64_t nVis = (t + 1) / 4;\n    expand_row(out, sortedIds"),
    "ids_fill_flat_iota": ("for (int64_t c = 0; c < numBlocks; ++c) ids[r * numBlocks + c] = (int32_t)c;",
                           "for (int64_t c = 0; c < numBlocks; ++c) ids[r * numBlocks + c] = (int32_t)(r * numBlocks + c);"),
    "ids_fill_from_one": ("for (int64_t c = 0; c < numBlocks; ++c) ids[r * numBlocks + c] = (int32_t)c;",
                          "for (int64_t c = 0; c < numBlocks; ++c) ids[r * numBlocks + c] = (int32_t)(c + 1);"),
    "rsqrt_single": ("float inv = (float)(1.0 / sqrt((double)v));",
                     "float inv = 1.0f / (float)sqrt((double)v) * (1.0f + 1.2e-7f);"),
}


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("mutants")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, mutant_dir):
    old, new = MUTANTS[name]
    assert SRC.count(old) >= 1, f"mutation site for {name} not found"
    src = SRC.replace(old, new)
    path = os.path.join(mutant_dir, f"{name}.c")
    open(path, "w").write(src)
    lib = os.path.join(mutant_dir, f"lib_{name}.so")
    import subprocess
    subprocess.run(["gcc", *obuild.FLAGS, "-Wno-error", path, "-o", lib, "-lm"], check=True)
    O = Oracle(lib)
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(O)
        except AssertionError:
            caught.append(check.__name__)
    O.set_threads(8)
    assert caught, f"no pin catches mutant {name}"
