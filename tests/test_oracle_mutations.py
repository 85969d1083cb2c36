"""Plant plausible mistakes in copies of the oracle; the pins must catch each one.

Each mutation edits the oracle's source text (on the CPU, in memory) and loads
it as a fresh module; the real oracle is untouched.
"""
import inspect
import types

import pytest

from oracle import sparse_decode_ref
from tests import pins

MUTATIONS = {
    "score_drops_last_term": ("for i in range(q.shape[0]):\n        acc = acc + q[i] * keys[:, i]",
                              "for i in range(q.shape[0] - 1):\n        acc = acc + q[i] * keys[:, i]"),
    "score_wrong_index": ("acc = acc + q[i] * keys[:, i]", "acc = acc + q[i] * keys[:, (i + 1) % q.shape[0]]"),
    "proxy_query_transposed": ("acc = acc + q[i] * P[i, :]", "acc = acc + q[i] * P[:, i % P.shape[1]][:P.shape[1]]"),
    "proxy_score_sign": ("acc = acc + qp[j] * Kp[:, j]", "acc = acc - qp[j] * Kp[:, j]"),
    "ties_to_higher_index": ("np.lexsort((np.arange(s.shape[0]), -s))", "np.lexsort((-np.arange(s.shape[0]), -s))"),
    "ascending_order": ("np.lexsort((np.arange(s.shape[0]), -s))", "np.lexsort((np.arange(s.shape[0]), s))"),
    "topk_off_by_one": ("order_desc(s)[: min(k, s.shape[0])]", "order_desc(s)[: min(k + 1, s.shape[0])]"),
    "topp_one_short": ("n_sel = int(hit[0]) + 1 if hit.size else n", "n_sel = max(1, int(hit[0])) if hit.size else n"),
    "topp_no_scale": ("ell = scale * s", "ell = s"),
    "topp_strict_gt_and_extra": ("hit = np.nonzero(c >= target)[0]", "hit = np.nonzero(c > target)[0] + 1"),
    "candidates_transposed": ("np.sort(segments)[:, None] * seg_size + np.arange(seg_size)[None, :]",
                              "np.sort(segments)[:, None] + np.arange(seg_size)[None, :] * seg_size"),
    "two_level_flat": ("pick = select_top_k(s2, k)", "pick = select_top_k(s2, k)[::-1][:1]"),
    "edge_off_by_one": ("b = np.arange(max(0, n - last), n)", "b = np.arange(max(0, n - last - 1), n)"),
    "attention_no_scale": ("logits = scale * (Kc @ qh.T)", "logits = (Kc @ qh.T)"),
    "attention_values_are_keys": ("o = (e.T @ Vc) / L[:, None]", "o = (e.T @ Kc) / L[:, None]"),
    "attention_lse_drops_max": ("return o, mx + np.log(L)\n\n\ndef lse_combine", "return o, np.log(L)\n\n\ndef lse_combine"),
    "combine_unweighted": ("o = (w[..., None] * o_parts).sum(axis=0) / L[..., None]", "o = o_parts.mean(axis=0)"),
    "hybrid_drops_summary": ("Kc = np.concatenate([Kc, src.Kg[bk, g][srows]], axis=0)", "Kc = Kc"),
    "hybrid_wrong_rows": ("(U[:, None] * chunk_size + np.arange(chunk_size)[None, :])",
                          "(U[:, None] + np.arange(chunk_size)[None, :])"),
    "forced_not_added": ("U = group_union([U, edge_entries(n_ent, w.keep_first, w.keep_last)])", "U = U"),
    "union_first_head_only": ("per_head.append(sel)", "per_head.append(sel) if not per_head else None"),
    "wrong_kv_group": ("qh = src.q[b, rows_q]\n", "qh = src.q[b, [(x + 1) % w.n_q_heads for x in rows_q]]\n"),
    "head_mask_drops_forced": ("S = group_union([heads[qi], forced])", "S = heads[qi]"),
    "head_mask_wrong_head": ("S = group_union([heads[qi], forced])", "S = group_union([heads[rows_q[(j + 1) % len(rows_q)]], forced])"),
    "multi_query_first_token_only": ("T = getattr(w, \"n_queries\", 1)\n    return", "T = 1\n    return"),
    "multi_query_rows_head_major": ("return [t * w.n_q_heads + g * G + j for t in range(T) for j in range(G)]",
                                    "return [(g * G + j) * T + t for t in range(T) for j in range(G)]"),
    "head_mask_ignored": ("masked = getattr(w, \"head_masks\", False) and", "masked = False and"),
    "coverage_cut_inclusive": ("hit = np.nonzero(c > thr)[0]", "hit = np.nonzero(c >= thr)[0] + 1"),
    "coverage_unnormalized": ("imp = imp + mass / math.fsum(mass.tolist())", "imp = imp + mass"),
    "coverage_descending": ("order = np.lexsort((-np.arange(n), imp))", "order = np.lexsort((-np.arange(n), -imp))"),
    "all_summaries_only_selected": ("srows = np.arange(n_ent) if all_sum else", "srows = np.asarray(S, dtype=np.int64) if all_sum else"),
    "growing_tail_dropped": ("tail = np.arange(n_ent * w.chunk_size, n_tok)", "tail = np.arange(0)"),
    "growing_scores_past_cache": ("s = chunk_scores(q, src.Kg[bk, g][:n_ent])\n            sel = select_top_k",
                                  "s = chunk_scores(q, src.Kg[bk, g])\n            sel = select_top_k"),
    "growing_forced_at_capacity": ("U = group_union([U, edge_entries(n_ent, w.keep_first, w.keep_last)])",
                                   "U = group_union([U, edge_entries(w.n_ctx // w.chunk_size, w.keep_first, w.keep_last)])"),
    "growing_proxy_past_cache": ("proxy_scores(qp, src.Kp[bk, g][:n_tok])", "proxy_scores(qp, src.Kp[bk, g])"),
    "growing_window_at_capacity": ("res[\"union\"] = edge_entries(n_ent, w.sink, w.window)",
                                   "res[\"union\"] = edge_entries(w.n_ctx // w.chunk_size, w.sink, w.window)"),
}


def _mutant(old, new):
    src = inspect.getsource(sparse_decode_ref)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    mod = _mutant(*MUTATIONS[name])
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # a failed assertion or a crash both count
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {name}"
