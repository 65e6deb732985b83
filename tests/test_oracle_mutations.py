"""Planted mistakes in the oracle must be caught by its pins.

Each case swaps one oracle helper for a copy carrying a plausible mistake (a
dropped term, a wrong index, a transposed operand, an off-by-one) and checks
that at least one pin from test_oracle_pins fails.  Everything runs on the
CPU; the real oracle is restored after each case.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import verify_oracle as O
from tests import test_oracle_hybrid as H
from tests import test_oracle_nested as N
from tests import test_oracle_pins as P
from tests import test_oracle_tree as T

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _fails(fn, *args) -> bool:
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def _tree_vis_without_self(kind, ids, lookback, _orig=O.block_visibility):
    vis = _orig(kind, ids, lookback)
    if kind == O.TREE:
        np.fill_diagonal(vis[1:, 1:], False)
    return vis


def _segment_lookback_off_by_one(kind, ids, lookback, _orig=O.block_visibility):
    if kind == O.SEGMENT and lookback > 0:
        return _orig(kind, ids, lookback - 1)
    return _orig(kind, ids, lookback)


def _gather_shifted(cache, block_row, ctx_len):
    out = np.empty((ctx_len,) + cache.shape[2:], dtype=np.float64)
    for t in range(ctx_len):
        tt = min(t + 1, ctx_len - 1)
        out[t] = cache[int(block_row[tt // O.PAGE]), tt % O.PAGE]
    return out


def _gather_slot_major(cache, block_row, ctx_len):
    out = np.empty((ctx_len,) + cache.shape[2:], dtype=np.float64)
    for t in range(ctx_len):
        out[t] = cache[int(block_row[t % O.PAGE]) if t % O.PAGE < len(block_row) else 0, t // O.PAGE]
    return out


def _attend_no_scale(q, keys, values, mask, scale, _orig=O.attend):
    return _orig(q, keys, values, mask, 1.0)


def _attend_values_are_keys(q, keys, values, mask, scale, _orig=O.attend):
    return _orig(q, keys, keys, mask, scale)


def _attend_lse_without_max(q, keys, values, mask, scale, _orig=O.attend):
    out, lse, p = _orig(q, keys, values, mask, scale)
    s = np.where(mask, scale * (q @ keys.T), -np.inf)
    return out, lse - s.max(axis=1), p


def _parents_self(kind, ids, _orig=O.acceptance_parents):
    par = _orig(kind, ids)
    if kind != O.TREE:
        par = np.arange(len(ids)) - 0  # compares row i with its own prediction
        par[0] = -1
    return par


def _targets_argmin(logits):
    return np.argmin(np.asarray(logits), axis=-1)


def _targets_last_on_ties(logits):
    lg = np.asarray(logits)
    V = lg.shape[-1]
    return (V - 1 - np.argmax(lg[..., ::-1], axis=-1)).astype(np.int64)


def _page_slot_swapped(block_row, t):
    return int(block_row[t // O.PAGE]), (t + 1) % O.PAGE


def _confidence_of_previous_row(draft_logits, draft_ids, _orig=O.draft_confidence):
    x = np.asarray(draft_logits)
    return _orig(np.concatenate([x[:, :1], x[:, :-1]], axis=1), draft_ids)


def _confidence_is_max_probability(draft_logits, draft_ids, _orig=O.draft_confidence):
    x = np.asarray(draft_logits)
    top = np.argmax(x, axis=-1)
    top[np.asarray(draft_ids) < 0] = -1
    return _orig(x, top)


def _hybrid_commits_h_drafts(draft_logits, logits, draft_ids, mask_kind, mask_ids, tau,
                             min_prefix, _orig=O.accept_hybrid):
    n, path, bonus, h = _orig(draft_logits, logits, draft_ids, mask_kind, mask_ids, tau,
                              min_prefix)
    hit = (h >= min_prefix) & (h >= 1)
    return np.where(hit, h, n), path, bonus, h


def _hybrid_strict_min_prefix(draft_logits, logits, draft_ids, mask_kind, mask_ids, tau,
                              min_prefix, _orig=O.accept_hybrid):
    return _orig(draft_logits, logits, draft_ids, mask_kind, mask_ids, tau, min_prefix + 1)


def _quantize_scale_over_8(x):
    x = np.asarray(x, dtype=np.float32)
    s = (np.abs(x).max(axis=-1) / np.float32(8.0)).astype(np.float32)
    live = s > 0
    t = (x / np.where(live, s, np.float32(1.0))[..., None]).astype(np.float32)
    q4 = np.clip(np.rint(t), -8, 7)
    qr = np.clip(np.rint(t * np.float32(16.0)) - 16.0 * q4, -8, 7)
    return (np.where(live[..., None], q4, 0).astype(np.int64),
            np.where(live[..., None], qr, 0).astype(np.int64), s)


def _quantize_half_away(x):
    x = np.asarray(x, dtype=np.float32)
    s = (np.abs(x).max(axis=-1) / np.float32(7.0)).astype(np.float32)
    live = s > 0
    t = (x / np.where(live, s, np.float32(1.0))[..., None]).astype(np.float32)
    q4 = np.sign(t) * np.floor(np.abs(t) + 0.5)
    qr = np.clip(np.sign(t) * np.floor(np.abs(16 * t) + 0.5) - 16.0 * q4, -8, 7)
    return (np.where(live[..., None], q4, 0).astype(np.int64),
            np.where(live[..., None], qr, 0).astype(np.int64), s)


def _pack_high_first(codes):
    u = (np.asarray(codes) + O.NEST_OFFSET).astype(np.uint8)
    return (u[..., 1::2] | (u[..., 0::2] << 4)).astype(np.uint8)


def _kv8_without_refinement(planes, level, _orig=O.dequantize_nested):
    return _orig(planes, 4)


def _refinement_grid_eighth(planes, level, _orig=O.dequantize_nested):
    if level != 8:
        return _orig(planes, level)
    q4 = O.unpack_nibbles(planes["base"]).astype(np.float64)
    qr = O.unpack_nibbles(planes["ref"]).astype(np.float64)
    s = np.asarray(planes["scale"], dtype=np.float64)[..., None]
    return (s * (8.0 * q4 + qr) / 8.0).transpose(0, 2, 1, 3)


def _recent_window_off_by_one(*args, kv8_recent=-1, _orig=O.verify_attention_nested, **kw):
    return _orig(*args, kv8_recent=kv8_recent + 1 if kv8_recent >= 0 else kv8_recent, **kw)


def _candidates_unpruned(p_row, parent_token):
    return sorted(range(len(p_row)), key=lambda v: (-float(p_row[v]), v))


def _candidates_ties_to_larger(p_row, parent_token):
    return sorted((v for v in range(len(p_row)) if v != parent_token),
                  key=lambda v: (-float(p_row[v]), -v))


def _mask_rows_from_root(probs, root_token, W, n_mask, min_cum_prob=0.0, _orig=O.dynamic_tree):
    d, par, dep, n = _orig(probs, root_token, W, n_mask, min_cum_prob)
    for b in range(len(n)):
        tail = 0
        for i in range(int(n[b]), W):
            par[b, i], dep[b, i], tail = tail, dep[b, tail] + 1, i
    return d, par, dep, n


MUTANTS = [
    ("block_visibility", _tree_vis_without_self, [(P.test_tree_visibility_is_ancestor_closure, 3),
                                                  (P.test_tree_golden_fixture,)]),
    ("block_visibility", _segment_lookback_off_by_one, [(P.test_lca_golden_fixture,)]),
    ("gather_committed", _gather_shifted, [(P.test_attention_matches_library_sdpa, "chain", -1, 0)]),
    ("gather_committed", _gather_slot_major, [(P.test_attention_matches_library_sdpa, "tree", -1, 1)]),
    ("attend", _attend_no_scale, [(P.test_attention_matches_library_sdpa, "tree", -1, 0)]),
    ("attend", _attend_values_are_keys, [(P.test_single_row_block_is_plain_decode_attention, 8, 2)]),
    ("attend", _attend_lse_without_max, [(P.test_equal_keys_average_the_visible_values, "chain")]),
    ("acceptance_parents", _parents_self, [(P.test_full_match_accepts_the_whole_chain,)]),
    ("target_ids", _targets_argmin, [(P.test_accept_golden_tree,)]),
    ("target_ids", _targets_last_on_ties, [(P.test_argmax_ties_take_the_smallest_id,)]),
    ("page_slot", _page_slot_swapped, [(P.test_commit_writes_exactly_the_accepted_rows, False)]),
    ("draft_confidence", _confidence_of_previous_row,
     [(H.test_confidence_is_the_softmax_probability_of_the_drafted_token,), (H.test_hybrid_golden_chain,)]),
    ("draft_confidence", _confidence_is_max_probability,
     [(H.test_confidence_is_the_softmax_probability_of_the_drafted_token,)]),
    ("accept_hybrid", _hybrid_commits_h_drafts, [(H.test_hybrid_golden_chain,),
                                                 (H.test_chain_confidence_prefix_closed_form, 0)]),
    ("accept_hybrid", _hybrid_strict_min_prefix, [(H.test_hybrid_golden_chain,)]),
    ("quantize_nested", _quantize_scale_over_8, [(N.test_golden_rows,),
                                                 (N.test_round_to_nearest_error_bounds, 0)]),
    ("quantize_nested", _quantize_half_away, [(N.test_golden_rows,)]),
    ("pack_nibbles", _pack_high_first, [(N.test_golden_rows,)]),
    ("dequantize_nested", _kv8_without_refinement,
     [(N.test_golden_rows,), (N.test_grid_exact_cache_reduces_to_dense_attention, "chain")]),
    ("dequantize_nested", _refinement_grid_eighth, [(N.test_golden_rows,)]),
    ("depth_candidates", _candidates_unpruned, [(T.test_golden_tree,)]),
    ("depth_candidates", _candidates_ties_to_larger, [(T.test_ties_go_to_the_smaller_token,)]),
    ("dynamic_tree", _mask_rows_from_root, [(T.test_golden_tree,)]),
    ("verify_attention_nested", _recent_window_off_by_one,
     [(N.test_recent_window_reads_kv8_only_for_the_newest_tokens,)]),
]


@pytest.mark.parametrize("name,mutant,pins", MUTANTS,
                         ids=[f"{n}:{m.__name__}" for n, m, _ in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, mutant, pins):
    monkeypatch.setattr(O, name, mutant)
    for pin in pins:
        assert _fails(pin[0], *pin[1:]), f"{pin[0].__name__} did not catch {mutant.__name__}"


def test_gqa_head_mapping_mistake_is_caught(monkeypatch):
    """Query head h reading KV head h % Hkv instead of h // group."""
    real = O.verify_attention

    def mutated(q, k_cache, v_cache, block_table, ctx_lens, k_new, v_new, mask_kind,
                mask_ids, scale=None, seg_lookback=-1):
        Hq, Hkv = q.shape[2], k_cache.shape[2]
        g = Hq // Hkv
        perm = np.array([(h % Hkv) * g + h // Hkv for h in range(Hq)])
        inv = np.argsort(perm)  # slot perm[h] of the real call carries head h
        out, lse = real(np.asarray(q)[:, :, inv], k_cache, v_cache, block_table, ctx_lens,
                        k_new, v_new, mask_kind, mask_ids, scale, seg_lookback)
        return out[:, :, perm], lse[:, :, perm]

    monkeypatch.setattr(O, "verify_attention", mutated)
    assert _fails(P.test_attention_matches_library_sdpa, "mixed", -1, 0)
