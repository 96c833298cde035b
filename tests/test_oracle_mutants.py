"""Plant plausible mistakes in copies of the oracle and check the pins catch each.

Every mutant is a textual patch of kascade_oracle.c compiled on the CPU into a
temporary library. All patches keep every memory access in bounds. A mutant
that no pin catches means the pins leave part of the oracle unchecked.
"""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle_pins  # noqa: E402

MUTANTS = {
    "pool_not_divided_by_G": (
        "for (int j = 0; j < N; ++j) pooled[j] /= nh;",
        "for (int j = 0; j < N; ++j) pooled[j] /= 1;"),
    "pool_first_head_only": (
        "*h0 = set * G;\n    *nh = G;",
        "*h0 = set * G;\n    *nh = 1;"),
    "shared_pools_one_group": (
        "*h0 = 0;\n    *nh = p->num_q_heads;",
        "*h0 = 0;\n    *nh = G;"),
    "shared_pools_first_kv_for_all_heads": (
        "s[j] = logit(p, q, k, b, h, 0, h / G, j);",
        "s[j] = logit(p, q, k, b, h, 0, p->shared_index_set ? 0 : h / G, j);"),
    "shared_reuse_ignores_batch": (
        "idx + ((size_t)b * index_sets(p) + set_of_head(p, h)) * K;",
        "idx + ((size_t)b * (p->shared_index_set ? 0 : index_sets(p)) + set_of_head(p, h)) * K;"),
    "shared_reuse_prefill_first_tile": (
        "idx + (((size_t)b * index_sets(p) + set_of_head(p, h)) * tiles + t) * K;",
        "idx + (((size_t)b * index_sets(p) + set_of_head(p, h)) * tiles + (p->shared_index_set ? 0 : t)) * K;"),
    "gqa_mapping_modulo": (
        "const int kvh = h / (p->num_q_heads / p->num_kv_heads), d = p->head_dim;",
        "const int kvh = h % p->num_kv_heads, d = p->head_dim;"),
    "reuse_prefill_excludes_diagonal": (
        "if (list[a] <= i) keys[nk++] = list[a];",
        "if (list[a] < i) keys[nk++] = list[a];"),
    "dense_causal_sees_next_key": (
        "int nk = causal ? i + 1 : N;",
        "int nk = causal ? (i + 2 < N ? i + 2 : N) : N;"),
    "ties_to_higher_index": (
        "return (x->j > y->j) - (x->j < y->j);",
        "return (x->j < y->j) - (x->j > y->j);"),
    "selects_smallest": (
        "if (x->value > y->value) return -1;\n  if (x->value < y->value) return 1;",
        "if (x->value > y->value) return 1;\n  if (x->value < y->value) return -1;"),
    "scale_dropped": (
        "return p->scale * acc;",
        "return acc;"),
    "k_read_as_v": (
        "out[c] += s[a] * element(v, p->dtype, vo + c);",
        "out[c] += s[a] * element(k, p->dtype, vo + c);"),
    "ragged_tile_divided_by_T": (
        "pooled[j] /= (double)nh * rows;",
        "pooled[j] /= (double)nh * T;"),
    "prefill_candidates_past_prefix": (
        "select_top_k(pooled, prefix, p->top_k,",
        "select_top_k(pooled, N, p->top_k,"),
    "reuse_prefill_wrong_tile": (
        "const int t = i / T;",
        "const int t = (i + 1) / T < tiles ? (i + 1) / T : tiles - 1;"),
    "softmax_not_normalised": (
        "for (int j = 0; j < n; ++j) s[j] /= l;",
        "for (int j = 0; j < n; ++j) s[j] /= 1.0;"),
    "lse_without_max": (
        "return m + log(l);",
        "return log(l);"),
    "bf16_widened_wrong": (
        "uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;",
        "uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 15;"),
    "tile_last_row_skipped": (
        "for (int i = row0; i < prefix; ++i) {",
        "for (int i = row0; i < prefix - 1; ++i) {"),
    "selection_not_sorted": (
        "qsort(out, (size_t)kt, sizeof *out, ascending);",
        "(void)ascending;"),
    "padding_zero": (
        "for (int s = kt; s < k; ++s) out[s] = -1;",
        "for (int s = kt; s < k; ++s) out[s] = 0;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    import oracle
    from oracle import build

    old, new = MUTANTS[name]
    src = build.read_source()
    assert src.count(old) == 1, f"patch target for {name} not found exactly once"
    lib = build.build_variant(src.replace(old, new), str(tmp_path))
    mutant = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"
