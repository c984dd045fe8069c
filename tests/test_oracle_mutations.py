"""Plant plausible mistakes in the oracle (on the CPU) and show a pin catches each.

A pin that no planted mistake can trip pins nothing; this file keeps the pin
set honest.  Every mutant is applied with monkeypatch and undone afterwards.
"""
import math

import numpy as np
import pytest

import _pins
import oracle.sparse_attn_oracle as O

_orig_softmax = O.softmax_attend
_orig_gather = O.gather_tokens
_orig_rank = O.rank_candidates
_orig_forced = O.forced_pages
_orig_union = O.gqa_union_block_table
_orig_summary = O.page_summary
_orig_sel_heads = O.selection_heads
_orig_row_pages = O.row_pages


def _no_scale(qrow, K, V, sm_scale, d_v):
    return _orig_softmax(qrow, K, V, 1.0, d_v)


def _no_max_shift(qrow, K, V, sm_scale, d_v):
    if K is None or K.shape[0] == 0:
        return np.zeros(d_v), -np.inf
    with np.errstate(over="ignore", invalid="ignore"):
        z = sm_scale * (K @ qrow)
        e = np.exp(z)
        l = e.sum()
        return (e @ V) / l, math.log(l) if np.isfinite(l) else float("nan")


def _v_not_transposed(k_pool, v_pool, block_table, b, g, pages, seq_len, page_size, d_v):
    """Read the page-transposed V pool as if it were token-major."""
    if v_pool is None:
        return _orig_gather(k_pool, v_pool, block_table, b, g, pages, seq_len, page_size, d_v)
    n, hk, dv, P = v_pool.shape
    token_major = np.ascontiguousarray(v_pool).reshape(n, hk, P, dv)
    return _orig_gather(k_pool, np.swapaxes(token_major, 2, 3), block_table, b, g, pages, seq_len,
                        page_size, d_v)


def _logical_as_physical(k_pool, v_pool, block_table, b, g, pages, seq_len, page_size, d_v):
    ident = np.tile(np.arange(block_table.shape[1], dtype=np.int32), (block_table.shape[0], 1))
    return _orig_gather(k_pool, v_pool, ident, b, g, pages, seq_len, page_size, d_v)


def _highest_index_ties(scores_row, candidates):
    """Break score ties toward the highest logical index."""
    def key(i):
        v = float(scores_row[i])
        return (1, 0.0, 0) if np.isnan(v) else (0, -v, -i)
    return sorted(candidates, key=key)


def _window_off_by_one(n, sink, window):
    return _orig_forced(n, sink, window + 1 if window > 0 else 0)


def _union_first_head_only(mask, n_kv):
    G = mask.shape[0] // n_kv
    return _orig_union(mask[::G].repeat(G, axis=0), n_kv)


def _summary_all_tokens(k_pool, block_table, seq_lens, page_size, last_pages=0):
    big = np.asarray(seq_lens) + page_size - 1
    full = (big // page_size) * page_size       # pretend every page is full
    return _orig_summary(k_pool, block_table, full, page_size, last_pages)


def _wrong_group(s, mode, group):
    heads, g = _orig_sel_heads(s, mode, group)
    return heads, (g + 1) % max(1, group) if mode == O.PER_Q_HEAD else g


def _ambient_ignores_mask(b, s, h, page_lists, page_counts, critical_counts, ambient_mask):
    return _orig_row_pages(b, s, h, page_lists, page_counts, None, None)


MUTANTS = {
    "no_softmax_scale": ("softmax_attend", _no_scale),
    "no_max_shift": ("softmax_attend", _no_max_shift),
    "v_read_untransposed": ("gather_tokens", _v_not_transposed),
    "logical_page_as_physical": ("gather_tokens", _logical_as_physical),
    "ties_to_highest_index": ("rank_candidates", _highest_index_ties),
    "window_off_by_one": ("forced_pages", _window_off_by_one),
    "union_skips_group_heads": ("gqa_union_block_table", _union_first_head_only),
    "mean_over_invalid_tokens": ("page_summary", _summary_all_tokens),
    "per_q_head_wrong_kv_head": ("selection_heads", _wrong_group),
    "ambient_mask_ignored": ("row_pages", _ambient_ignores_mask),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for check in _pins.ALL_CHECKS:
        try:
            check()
        except Exception as e:  # AssertionError, or a shape error the mistake causes
            caught.append((check.__name__, type(e).__name__))
    assert caught, f"planted mistake {name} passed every pin"
