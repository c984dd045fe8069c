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
_orig_mask = O.prefill_block_mask
_orig_fp8 = O.fp8_e4m3_to_float
_orig_deq = O.dequantize_pages
_orig_mc = O.mean_corrected_prefill
_orig_mass = O.head_page_mass
_orig_beta = O.tier_beta
_orig_cov = O.tier_coverage


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


def _latent_v_from_tail(k_pool, v_pool, block_table, b, g, pages, seq_len, page_size, d_v):
    """Latent cache: take V from the last d_v dims of the row (rope dims included)."""
    K, V = _orig_gather(k_pool, v_pool, block_table, b, g, pages, seq_len, page_size, d_v)
    if v_pool is None and K is not None:
        V = K[:, -d_v:]
    return K, V


def _latent_k_head_only(k_pool, v_pool, block_table, b, g, pages, seq_len, page_size, d_v):
    """Latent cache: score against the first d_v dims only (rope dims dropped from K)."""
    K, V = _orig_gather(k_pool, v_pool, block_table, b, g, pages, seq_len, page_size, d_v)
    if v_pool is None and K is not None:
        K = np.concatenate([K[:, :d_v], np.zeros_like(K[:, d_v:])], axis=1)
    return K, V


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


def _mask_sum_not_mean(q, mu, bt, seq_len, P, q_start, bq, nkb, n_kv, scale, top_k=None, max_gap=None):
    """Pool the Q-block's queries by their sum instead of their mean."""
    qs = np.array(q, dtype=np.float64)
    for qb in range(0, qs.shape[0], bq):
        qs[qb:qb + bq] *= min(bq, qs.shape[0] - qb)
    return _orig_mask(qs, mu, bt, seq_len, P, q_start, bq, nkb, n_kv, scale, top_k=top_k, max_gap=max_gap)


def _mask_no_diagonal(q, mu, bt, seq_len, P, q_start, bq, nkb, n_kv, scale, top_k=None, max_gap=None):
    """Forget to force the diagonal block of each Q-block."""
    m, sc = _orig_mask(q, mu, bt, seq_len, P, q_start, bq, nkb, n_kv, scale, top_k=top_k, max_gap=max_gap)
    m = m.copy()
    for qb in range(m.shape[1]):
        last = q_start + min((qb + 1) * bq, q.shape[0]) - 1
        if last // P > 0:
            m[:, qb, last // P] = 0
    return m, sc


def _mask_one_past_causal(q, mu, bt, seq_len, P, q_start, bq, nkb, n_kv, scale, top_k=None, max_gap=None):
    """Let each Q-block also keep the block just past its last query."""
    m, sc = _orig_mask(q, mu, bt, seq_len, P, q_start, bq, nkb, n_kv, scale, top_k=top_k, max_gap=max_gap)
    m = m.copy()
    for qb in range(m.shape[1]):
        nxt = (q_start + min((qb + 1) * bq, q.shape[0]) - 1) // P + 1
        if nxt < nkb:
            m[:, qb, nxt] = 1
    return m, sc


def _fp8_bias_8(codes):
    """Decode E4M3 with exponent bias 8 (the FNUZ variant's bias)."""
    return _orig_fp8(codes) / 2.0


def _fp8_no_subnormals(codes):
    """Flush exponent-0 codes to zero."""
    c = np.asarray(codes, dtype=np.int64)
    v = _orig_fp8(codes)
    return np.where(((c >> 3) & 0xF) == 0, 0.0 * v, v)


def _deq_scale_ignored(pool, scale):
    return _orig_deq(pool, np.ones_like(scale))


def _mc_no_count(q, kp, vp, bt, L, P, q_start, tables, counts, n_kv, scale, rows=None):
    """Weight each skipped block as a single token (its count n_b left out)."""
    q_len, Hq, d = q.shape
    G = Hq // n_kv
    out = np.zeros((q_len, Hq, vp.shape[2]))
    lse = np.full((q_len, Hq), np.nan)
    for i in range(q_len):
        for h in range(Hq):
            g, pos = h // G, q_start + i
            table = set(int(x) for x in tables[g, :int(counts[g])])
            zs, vs = [], []
            for kb in range(O.n_pages_of(L, P)):
                nv = O.valid_tokens(L, kb, P)
                K = np.asarray(kp[int(bt[kb]), g, :nv], dtype=np.float64)
                V = np.asarray(vp[int(bt[kb]), g, :, :nv], dtype=np.float64).T
                if kb in table:
                    for r in range(nv):
                        if kb * P + r <= pos:
                            zs.append(scale * float(q[i, h] @ K[r]))
                            vs.append(V[r])
                elif kb * P + nv - 1 <= pos:
                    zs.append(scale * float(q[i, h] @ K.mean(axis=0)))
                    vs.append(V.mean(axis=0))
            z = np.array(zs)
            e = np.exp(z - z.max())
            out[i, h] = (e @ np.stack(vs)) / e.sum()
            lse[i, h] = z.max() + math.log(e.sum())
    return out, lse


def _mc_partial_blocks(q, kp, vp, bt, L, P, q_start, tables, counts, n_kv, scale, rows=None):
    """Also count skipped blocks that are only partly visible (their later tokens past the query)."""
    return _orig_mc(q, kp, vp, bt, L, P, q_start + P - 1, tables, counts, n_kv, scale, rows)


def _mass_no_count(q, mu, block_table, seq_lens, page_size, n_kv_heads, sm_scale):
    """Page log-weights without the ln n_p term (a partial page weighs like a full one)."""
    B, T, Hq, d = q.shape
    G = Hq // n_kv_heads
    M = np.full((B, Hq, block_table.shape[1]), np.nan)
    for b in range(B):
        n = O.n_pages_of(seq_lens[b], page_size)
        M[b, :, :n] = 0.0
        for h in range(Hq):
            mus = np.stack([np.asarray(mu[int(block_table[b, p]), h // G], dtype=np.float64) for p in range(n)])
            for t in range(T):
                est = sm_scale * (mus @ np.asarray(q[b, t, h], dtype=np.float64))
                e = np.exp(est - est.max())
                M[b, h, :n] += e / e.sum()
    return M


def _mass_no_scale(q, mu, block_table, seq_lens, page_size, n_kv_heads, sm_scale):
    return _orig_mass(q, mu, block_table, seq_lens, page_size, n_kv_heads, 1.0)


def _beta_plus_one(alpha, h, budget, group):
    b = _orig_beta(alpha, h, budget, group)
    return None if b is None else b + 1


def _top_heads_lowest(masses, heads, h):
    order = sorted(heads, key=lambda x: (float(masses[x]), x))
    return sorted(order[:max(0, min(h, len(order)))])


def _top_heads_ties_high(masses, heads, h):
    order = sorted(heads, key=lambda x: (-float(masses[x]), -x))
    return sorted(order[:max(0, min(h, len(order)))])


def _cov_no_forced(M, scores, seq_lens, P, n_kv, T, sink, window, budget, alphas, hs):
    return _orig_cov(M, scores, seq_lens, P, n_kv, T, 0, 0, budget, alphas, hs)


MUTANTS = {
    "mass_no_log_count": ("head_page_mass", _mass_no_count),
    "mass_no_scale": ("head_page_mass", _mass_no_scale),
    "tier_beta_plus_one": ("tier_beta", _beta_plus_one),
    "ambient_heads_lowest_mass": ("top_heads", _top_heads_lowest),
    "ambient_heads_ties_high_index": ("top_heads", _top_heads_ties_high),
    "coverage_drops_forced_pages": ("tier_coverage", _cov_no_forced),
    "mean_correction_no_count": ("mean_corrected_prefill", _mc_no_count),
    "mean_correction_partial_blocks": ("mean_corrected_prefill", _mc_partial_blocks),
    "fp8_bias_8": ("fp8_e4m3_to_float", _fp8_bias_8),
    "fp8_no_subnormals": ("fp8_e4m3_to_float", _fp8_no_subnormals),
    "fp8_page_scale_ignored": ("dequantize_pages", _deq_scale_ignored),
    "mask_sum_not_mean": ("prefill_block_mask", _mask_sum_not_mean),
    "mask_no_diagonal": ("prefill_block_mask", _mask_no_diagonal),
    "mask_one_past_causal": ("prefill_block_mask", _mask_one_past_causal),
    "no_softmax_scale": ("softmax_attend", _no_scale),
    "no_max_shift": ("softmax_attend", _no_max_shift),
    "v_read_untransposed": ("gather_tokens", _v_not_transposed),
    "logical_page_as_physical": ("gather_tokens", _logical_as_physical),
    "latent_v_from_tail": ("gather_tokens", _latent_v_from_tail),
    "latent_k_drops_rope": ("gather_tokens", _latent_k_head_only),
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
