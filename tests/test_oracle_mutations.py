"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of an oracle function (its source with
one edit, compiled in the oracle module's namespace), swaps the copy in, and
runs the pins named for that function: at least one of them must fail.  The
planted copies exist only inside this test, on the CPU; the oracle itself is
restored after every case.
"""
import inspect
import textwrap

import pytest

from oracle import lsa_oracle as O
from oracle import scan_oracle as SO

import test_oracle_pins as P
import test_oracle_tree_pins as TP
import test_scan_oracle_pins as SP
import test_oracle_near_pins as NP


def _module(fn_name: str):
    return SO if fn_name.startswith(("scan_", "run_")) else O


def _broken(fn_name: str, old: str, new: str):
    mod = _module(fn_name)
    src = textwrap.dedent(inspect.getsource(getattr(mod, fn_name)))
    assert src.count(old) == 1, f"{fn_name}: the text to break is not found once: {old!r}"
    ns = dict(vars(mod))
    exec(compile(src.replace(old, new), f"<broken {fn_name}>", "exec"), ns)
    return ns[fn_name]


TREE_RANK_PINS = [TP.test_fixed_level_search_scores_every_node_of_its_start_level,
                  TP.test_tree_rank_beam1_follows_the_parent_not_the_best_bucket,
                  TP.test_tree_rank_beam2_three_levels,
                  TP.test_tree_rank_tie_at_the_beam_boundary_keeps_the_lower_node,
                  TP.test_tree_rank_masks_subtrees_with_no_eligible_block,
                  TP.test_tree_rank_leaf_phase_drops_ineligible_buckets]
BUILD_TREE_PINS = [TP.test_build_tree_parent_centroid_is_the_rounded_unit_sum,
                   TP.test_build_tree_one_child_parent_copies_its_child_bit_for_bit,
                   TP.test_build_tree_pairs_only_inside_groups_of_128]

SCAN_PINS = [SP.test_worked_query_scan_counts, SP.test_block_scan_hand_worked,
             SP.test_run_direction_is_the_normalised_mean_of_unit_keys,
             SP.test_token_scan_takes_the_k_best_far_keys,
             SP.test_scan_with_k_covering_every_key_is_dense_causal]

NEAR_PINS = [NP.test_near_union_hand_worked, NP.test_near_union_clips_sinks_to_the_query,
             NP.test_near_union_count_limits_the_list,
             NP.test_near_union_window_only_query_near_start]

MUTATIONS = [
    # near_union
    ("near_union", "if 0 <= e < T and int(e) not in near_s]", "if 0 <= e < T]",
     "near entries of the list counted twice", NEAR_PINS),
    ("near_union", "np.asarray(idx[:count]).tolist()", "np.asarray(idx).tolist()",
     "entries past the count read", NEAR_PINS),
    ("near_union", "if 0 <= e < T and int(e) not in near_s]", "if int(e) not in near_s]",
     "invalid entries kept", NEAR_PINS),
    # tree_rank
    ("tree_rank", "o = np.lexsort((kids, -sc))", "o = np.lexsort((kids, sc))",
     "beam keeps the lowest scores", TREE_RANK_PINS),
    ("tree_rank", "o = np.lexsort((kids, -sc))", "o = np.lexsort((-kids, -sc))",
     "beam ties go to the higher node", TREE_RANK_PINS),
    ("tree_rank", 'kids = kids[here["min_block"][kids] < qb]', "kids = kids",
     "no causal mask on tree nodes", TREE_RANK_PINS),
    ("tree_rank", 'kids = kids[here["min_block"][kids] < qb]',
     'kids = kids[here["min_block"][kids] <= qb]', "mask admits the query's own block",
     TREE_RANK_PINS),
    ("tree_rank", "nodes = nodes[nodes < eligible_buckets(p, prm)]", "nodes = nodes",
     "leaf phase keeps ineligible buckets", TREE_RANK_PINS),
    ("tree_rank", "range(S - 1, lstar - 1, -1)", "range(S - 1, lstar, -1)",
     "beam stops one level early", TREE_RANK_PINS),
    ("tree_rank", "beam = np.sort(kids[o[:prm.beam]])", "beam = np.sort(kids[o[:prm.beam + 1]])",
     "beam one wider", TREE_RANK_PINS),
    ("tree_rank", "o = np.lexsort((nodes, -sc))", "o = np.lexsort((nodes, sc))",
     "leaf phase ranks worst first", TREE_RANK_PINS),
    ("tree_rank", "S = H if prm.start_level < 0 else min(max(prm.start_level, lstar), H)", "S = H",
     "start level ignored", TREE_RANK_PINS),
    ("tree_rank", 'nodes = np.flatnonzero(lv["min_block"] < qb)',
     'nodes = np.arange(lv["cent"].shape[0])', "first stage without the causal mask",
     TREE_RANK_PINS + [TP.test_fixed_level_search_masks_ineligible_nodes]),
    # build_tree
    ("build_tree", 'cent.append(round_index(unit(below["cent"][kids].sum(axis=0)), dtype))',
     'cent.append(round_index(below["cent"][kids].mean(axis=0), dtype))',
     "parent = rounded mean of the children", BUILD_TREE_PINS),
    ("build_tree", 'cent.append(round_index(unit(below["cent"][kids].sum(axis=0)), dtype))',
     'cent.append(unit(below["cent"][kids].sum(axis=0)))',
     "parent centroid not rounded", BUILD_TREE_PINS),
    ("build_tree", 'cent.append(below["cent"][kids[0]].copy())',
     'cent.append(round_index(unit(below["cent"][kids[0]]), dtype))',
     "one-child parent renormalised", BUILD_TREE_PINS),
    ("build_tree", 'minb.append(below["min_block"][kids].min())',
     'minb.append(below["min_block"][kids].max())', "min_block takes the largest block",
     BUILD_TREE_PINS),
    ("build_tree", "for c in res.clusters:", "for c in sorted(res.clusters, key=max):",
     "parents ordered by their larger child", BUILD_TREE_PINS),
    ("build_tree", "min(n, g0 + TREE_GROUP)", "n", "pairing across the whole level",
     BUILD_TREE_PINS),
    # the bucket bound
    ("leaf_level", "while prm.beam * (1 << l) < prm.top_b:",
     "while prm.beam * (1 << l) < -(-prm.k // prm.n_pool) + 65:",
     "l* from the default-window bound", [P.test_leaf_level_reading,
                                           TP.test_top_b_reading_by_hand]),
    # rounding, normalisation, the Ward cost, the decode trigger
    ("round_bf16", "return np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)",
     "return np.ldexp(np.floor(np.ldexp(x, 8 - e)), e - 8)", "bf16 rounding truncates",
     [P.test_round_bf16_matches_torch_nearest_even, P.test_normalize_query_by_hand]),
    ("normalize_query", "return round_index(unit(np.asarray(y, np.float64)), dtype)",
     "return round_index(np.asarray(y, np.float64), dtype)", "query not normalised",
     [P.test_normalize_query_by_hand]),
    ("ward_cost", "return n_a * n_b / (n_a + n_b) * float(np.dot(d, d))",
     "return float(np.dot(d, d))", "Ward cost without the size factor",
     [P.test_ward_cost_equals_brute_force_ess_increase]),
    ("decode_fires", "return (p + 1) % prm.block == 0", "return p % prm.block == 0",
     "block fires on its first key", [P.test_decode_fires_when_a_block_fills]),
    # sinks, expansion order, the cache's centroids and key numbering
    ("near_set", "sinks = np.arange(min(prm.n_sink, p + 1))", "sinks = np.arange(prm.n_sink)",
     "sinks not clipped to the query", NEAR_PINS),
    ("expand", "if len(far) == k:", "if len(far) == k + 1:", "one far key too many",
     [P.test_expansion_worked_example_by_hand]),
    ("build_cache", "cent[g] = round_index(unit(s), prm.index_dtype)",
     "cent[g] = round_index(unit(P[c].mean(axis=0) * 0 + P[c][0]), prm.index_dtype)",
     "centroid from the first member only", [P.test_centroid_is_normalised_sum_of_member_unit_keys]),
    ("build_cache", "members[g] = [b * prm.block + prm.n_pool * j + i",
     "members[g] = [b * prm.block + j + i", "members numbered by item, not key",
     [P.test_bucket_partition_invariants_and_counts]),
    # max over query heads (N-LSA scoring)
    ("bucket_scores", "return (cent @ yhat.T).max(axis=1)", "return (cent @ yhat.T).mean(axis=1)",
     "heads averaged instead of maxed", [P.test_max_over_heads_bucket_scores_hand_worked,
                                         P.test_max_over_heads_lists_by_hand]),
    ("bucket_scores", "return (cent @ yhat.T).max(axis=1)", "return cent @ yhat[0]",
     "first head only", [P.test_max_over_heads_bucket_scores_hand_worked,
                         P.test_max_over_heads_lists_by_hand]),
    # flat ranking, expansion, near set, Ward, attention
    ("flat_rank", "order = np.lexsort((np.arange(ne), -s))",
     "order = np.lexsort((-np.arange(ne), -s))", "flat ties to the higher bucket",
     [P.test_flat_rank_ties_go_to_lower_bucket]),
    ("eligible_buckets", "prm.n_buckets * (p // prm.block)",
     "prm.n_buckets * (p // prm.block + 1)", "query's own block eligible",
     [P.test_worked_query_counts_from_the_pages]),
    ("near_set", "win = np.arange(max(0, p - prm.window + 1), p + 1)",
     "win = np.arange(max(0, p - prm.window), p + 1)", "window of 513 keys",
     [P.test_worked_query_counts_from_the_pages]),
    ("expand", "if key not in near_s:", "if True:", "sinks and window not skipped",
     [P.test_expansion_worked_example_by_hand]),
    ("ward_merge", "flat = int(np.argmin(vals))",
     "flat = int(len(vals) - 1 - np.argmin(vals[::-1]))", "Ward ties to the largest pair",
     [P.test_ward_respects_cap_and_tie_rule]),
    ("ward_merge", "(size[:, None] + size[None, :]) <= cap)",
     "(size[:, None] + size[None, :]) <= cap + 1)", "size cap one too large",
     [P.test_bucket_partition_invariants_and_counts]),
    ("attention_query", "logits = (Kh @ q[h]) * scale", "logits = (Kh @ q[h])",
     "attention scale dropped", [P.test_attention_with_full_list_equals_dense_causal_sdpa]),
    ("attention_query", "hk = h * Hkv // Hq", "hk = h % Hkv", "GQA heads interleaved",
     [P.test_attention_with_full_list_equals_dense_causal_sdpa]),
    ("pool_keys", "return Khat[:T].reshape(-1, n_pool, Khat.shape[1]).sum(axis=1)",
     "return Khat[:T].reshape(-1, n_pool, Khat.shape[1]).mean(axis=1)", "pooled mean, not sum",
     [P.test_normalise_and_pool_are_sums_of_unit_keys]),
    # the scan baselines
    ("scan_runs", "j_hi = w_start // b", "j_hi = -(-w_start // b)",
     "scan includes the run that straddles the window", SCAN_PINS),
    ("scan_runs", "j_lo = s_end // b", "j_lo = 0", "scan counts sink-only runs", SCAN_PINS),
    ("scan_rank", "order = np.lexsort((runs, -s))", "order = np.lexsort((-runs, -s))",
     "scan ties to the higher run", SCAN_PINS),
    ("scan_rank", "order = np.lexsort((runs, -s))", "order = np.lexsort((runs, s))",
     "scan opens the worst runs first", SCAN_PINS),
    ("scan_expand", "if key not in near_s:", "if True:", "scan takes sink keys", SCAN_PINS),
    ("run_directions", "return unit(normalize_keys(X[:n]).reshape(-1, b, X.shape[1]).sum(axis=1))",
     "return unit(X[:n].reshape(-1, b, X.shape[1]).sum(axis=1))",
     "run summary of raw (not unit) keys", SCAN_PINS),
]


@pytest.mark.parametrize("fn,old,new,what,pins", MUTATIONS, ids=[m[3] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(fn, old, new, what, pins, monkeypatch):
    # every pin runs without arguments (a call that fails for want of them
    # would count as a catch)
    for pin in pins:
        assert not any(p.default is inspect.Parameter.empty
                       for p in inspect.signature(pin).parameters.values()), pin.__name__
    monkeypatch.setattr(_module(fn), fn, _broken(fn, old, new))
    failed = []
    for pin in pins:
        try:
            pin()
        except Exception as e:          # an assertion or a crash: the pin caught it
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"no pin catches: {what}"
