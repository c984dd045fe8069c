"""Checks that pin the CPU oracle to things other than itself.

Each ``check_*`` raises AssertionError on failure.  They are run as tests in
test_oracle_pins.py and, with mistakes planted into the oracle, in
test_oracle_mutations.py (each planted mistake must trip at least one check).

Independent references used here:
  * pure-Python brute force (``sorted`` with an explicit key, ``math.fsum``,
    explicit set unions) on tiny inputs;
  * torch's scaled_dot_product_attention / logsumexp in float64 on the CPU,
    over dense K/V that the test scatters into a shuffled paged pool itself;
  * closed forms (constant V, single token, integer-exact scores);
  * hand-derived golden cases under tests/golden/.
"""
from __future__ import annotations

import json
import math
import os
import random

import numpy as np
import torch

import oracle.sparse_attn_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------------ helpers
def scatter_to_pool(K, V, page_size, rng, extra_pages=0):
    """Dense K [B][Hkv][L][d], V [B][Hkv][L][dv] -> shuffled paged pool.

    Returns (k_pool [n_phys][Hkv][P][d], v_pool [n_phys][Hkv][dv][P],
    block_table [B][max_pages]).  Written as a direct scatter, independent of
    the oracle's gather.
    """
    B, Hkv, L, d = K.shape
    dv = V.shape[-1]
    P = page_size
    npg = (L + P - 1) // P
    n_phys = B * npg + extra_pages
    perm = rng.permutation(n_phys)
    kp = rng.standard_normal((n_phys, Hkv, P, d)) * 1e3      # junk where no token lands
    vp = rng.standard_normal((n_phys, Hkv, dv, P)) * 1e3
    bt = np.full((B, npg), -1, dtype=np.int32)
    for b in range(B):
        for lp in range(npg):
            phys = int(perm[b * npg + lp])
            bt[b, lp] = phys
            for r in range(P):
                j = lp * P + r
                if j >= L:
                    continue
                for g in range(Hkv):
                    kp[phys, g, r, :] = K[b, g, j, :]
                    vp[phys, g, :, r] = V[b, g, j, :]
    return kp, vp, bt


def sdpa(qrows, K, V, scale, allowed):
    """torch float64 SDPA + logsumexp for query rows [n][d] over K [L][d], V [L][dv], mask [n][L]."""
    qt = torch.from_numpy(np.asarray(qrows, dtype=np.float64))[None, None]
    kt = torch.from_numpy(np.asarray(K, dtype=np.float64))[None, None]
    vt = torch.from_numpy(np.asarray(V, dtype=np.float64))[None, None]
    mt = torch.from_numpy(np.asarray(allowed, dtype=bool))[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt, scale=scale)[0, 0]
    z = scale * (qt[0, 0] @ kt[0, 0].T)
    z = z.masked_fill(~mt[0, 0], float("-inf"))
    lse = torch.logsumexp(z, dim=-1)
    return o.numpy(), lse.numpy()


def _lists_from(sel_sets, stride):
    B = len(sel_sets)
    S = len(sel_sets[0])
    lists = np.full((B, S, stride), -1, dtype=np.int32)
    counts = np.zeros((B, S), dtype=np.int32)
    for b in range(B):
        for s in range(S):
            ls = sorted(sel_sets[b][s])
            lists[b, s, :len(ls)] = ls
            counts[b, s] = len(ls)
    return lists, counts


# -------------------------------------------------------------------- a0
def check_summary_constant_pages():
    rng = np.random.default_rng(1)
    B, Hkv, P, d, L = 2, 2, 4, 3, 10
    K = np.zeros((B, Hkv, L, d))
    for b in range(B):
        for lp in range(3):
            for g in range(Hkv):
                K[b, g, lp * P:(lp + 1) * P, :] = (b + 1) * 10 + lp + 0.25 * g
    kp, _, bt = scatter_to_pool(K, K, P, rng)
    mu = O.page_summary(kp, bt, np.array([L, L]), P)
    for b in range(B):
        for lp in range(3):
            for g in range(Hkv):
                exp = (b + 1) * 10 + lp + 0.25 * g
                assert np.all(mu[bt[b, lp], g] == np.float32(exp)), (b, lp, g)


def check_summary_bruteforce():
    rng = np.random.default_rng(2)
    B, Hkv, P, d = 2, 2, 4, 5
    lens = [11, 6]
    L = max(lens)
    K = rng.standard_normal((B, Hkv, L, d))
    kp, _, bt = scatter_to_pool(K, K, P, rng)
    mu = O.page_summary(kp, bt, np.array(lens), P)
    for b in range(B):
        for lp in range((lens[b] + P - 1) // P):
            toks = [j for j in range(lp * P, (lp + 1) * P) if j < lens[b]]
            for g in range(Hkv):
                for e in range(d):
                    exp = math.fsum(K[b, g, j, e] for j in toks) / len(toks)
                    got = float(mu[bt[b, lp], g, e])
                    assert abs(got - exp) <= 1e-6 * max(1.0, abs(exp)), (b, lp, g, e, got, exp)
    # last_pages=1 touches only each sequence's last page
    mu1 = O.page_summary(kp, bt, np.array(lens), P, last_pages=1)
    for b in range(B):
        n = (lens[b] + P - 1) // P
        for lp in range(n):
            touched = not np.isnan(mu1[bt[b, lp]]).any()
            assert touched == (lp == n - 1)


# -------------------------------------------------------------------- a1
def check_scores_exact_integers():
    """Small integers make every sum exact: compare with integer arithmetic."""
    rng = np.random.default_rng(3)
    B, T, Hq, Hkv, P, d, L = 2, 2, 4, 2, 4, 6, 16
    q = rng.integers(-3, 4, size=(B, T, Hq, d)).astype(np.float64)
    K = rng.integers(-4, 5, size=(B, Hkv, L, d)).astype(np.float64)
    kp, _, bt = scatter_to_pool(K, K, P, rng)
    mu = O.page_summary(kp, bt, np.array([L] * B), P)
    G = Hq // Hkv
    for mode in (O.PER_KV_HEAD, O.PER_Q_HEAD):
        sc = O.page_scores(q, mu, bt, np.array([L] * B), P, Hkv, mode)
        S = Hkv if mode == O.PER_KV_HEAD else Hq
        for b in range(B):
            for s in range(S):
                heads = list(range(s * G, (s + 1) * G)) if mode == O.PER_KV_HEAD else [s]
                g = s if mode == O.PER_KV_HEAD else s // G
                for lp in range(L // P):
                    num = 0
                    for e in range(d):
                        qs = sum(int(q[b, t, h, e]) for t in range(T) for h in heads)
                        ks = sum(int(K[b, g, j, e]) for j in range(lp * P, (lp + 1) * P))
                        num += qs * ks
                    assert float(sc[b, s, lp]) == num / P, (mode, b, s, lp)


def check_scores_linearity_and_unfactored():
    """Group score = sum of the group's per-head scores = mean over tokens of sum_{t,h} q.k_j."""
    rng = np.random.default_rng(4)
    B, T, Hq, Hkv, P, d = 2, 2, 6, 2, 8, 16
    lens = [37, 24]
    L = max(lens)
    q = rng.standard_normal((B, T, Hq, d))
    K = rng.standard_normal((B, Hkv, L, d))
    kp, _, bt = scatter_to_pool(K, K, P, rng)
    mu = O.page_summary(kp, bt, np.array(lens), P)
    sg = O.page_scores(q, mu, bt, np.array(lens), P, Hkv, O.PER_KV_HEAD)
    sq = O.page_scores(q, mu, bt, np.array(lens), P, Hkv, O.PER_Q_HEAD)
    G = Hq // Hkv
    for b in range(B):
        n = (lens[b] + P - 1) // P
        for g in range(Hkv):
            for lp in range(n):
                per_head = math.fsum(float(sq[b, h, lp]) for h in range(g * G, (g + 1) * G))
                assert abs(float(sg[b, g, lp]) - per_head) <= 1e-5 * (1 + abs(per_head))
                toks = [j for j in range(lp * P, (lp + 1) * P) if j < lens[b]]
                unf = math.fsum(float(q[b, t, h] @ K[b, g, j]) for j in toks for t in range(T)
                                for h in range(g * G, (g + 1) * G)) / len(toks)
                assert abs(float(sg[b, g, lp]) - unf) <= 1e-5 * (1 + abs(unf)), (b, g, lp)
    # pages past the end of a sequence carry no score
    assert np.isnan(sg[1, :, 3:]).all()


# -------------------------------------------------------------------- a2
def _brute_select(scores, n, sink, window, top_k, critical_k):
    forced = sorted(set(range(min(sink, n))) | set(range(max(0, n - window), n)))
    cand = [i for i in range(n) if i not in forced]

    def key(i):
        s = float(scores[i])
        return (1, 0.0, i) if math.isnan(s) else (0, -s, i)

    ranked = sorted(cand, key=key)
    k = min(max(top_k, 0), len(ranked))
    chosen = ranked[:k]
    if critical_k is None:
        return sorted(set(forced) | set(chosen)), None
    ck = min(critical_k, k)
    crit = sorted(set(forced) | set(chosen[:ck]))
    return crit + sorted(chosen[ck:]), len(crit)


def check_select_bruteforce():
    rng = np.random.default_rng(5)
    for trial in range(60):
        B, S = 2, 3
        n_pages = [int(rng.integers(1, 40)), int(rng.integers(1, 40))]
        mp = max(n_pages)
        # few distinct values -> many exact ties; a few NaNs and signed zeros
        scores = rng.integers(-3, 4, size=(B, S, mp)).astype(np.float32)
        scores[rng.random((B, S, mp)) < 0.05] = np.nan
        scores[rng.random((B, S, mp)) < 0.05] = -0.0
        sink, window = int(rng.integers(0, 4)), int(rng.integers(0, 6))
        top_k = int(rng.integers(0, 45))
        critical_k = None if trial % 2 == 0 else int(rng.integers(0, top_k + 2))
        lists, counts, cc = O.select_pages(scores, n_pages, sink, window, top_k, critical_k)
        for b in range(B):
            for s in range(S):
                exp, ecc = _brute_select(scores[b, s], n_pages[b], sink, window, top_k, critical_k)
                got = [int(x) for x in lists[b, s, :counts[b, s]]]
                assert got == exp, (trial, b, s, got, exp)
                assert (lists[b, s, counts[b, s]:] == -1).all()
                if critical_k is not None:
                    assert int(cc[b, s]) == ecc


def check_select_golden():
    with open(os.path.join(GOLDEN, "select_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        sc = np.array([float(x) for x in c["scores"]], dtype=np.float32)[None, None, :]
        lists, counts, cc = O.select_pages(sc, [sc.shape[-1]], c["sink"], c["window"], c["top_k"],
                                           c["critical_k"])
        got = [int(x) for x in lists[0, 0, :counts[0, 0]]]
        assert got == c["list"], (c["name"], got, c["list"])
        if c["critical_count"] is not None:
            assert int(cc[0, 0]) == c["critical_count"], c["name"]


# ----------------------------------------------------------------- a3-a5
def _dense_decode_case(rng, B=2, T=2, Hq=4, Hkv=2, P=4, d=8, dv=8, lens=(19, 12)):
    L = max(lens)
    q = rng.standard_normal((B, T, Hq, d))
    K = rng.standard_normal((B, Hkv, L, d))
    V = rng.standard_normal((B, Hkv, L, dv))
    kp, vp, bt = scatter_to_pool(K, V, P, rng, extra_pages=3)
    return q, K, V, kp, vp, bt, np.array(lens)


def check_decode_select_all_sdpa():
    rng = np.random.default_rng(6)
    q, K, V, kp, vp, bt, lens = _dense_decode_case(rng)
    B, T, Hq, d = q.shape
    Hkv, P = K.shape[1], 4
    G = Hq // Hkv
    sets = [[set(range((int(lens[b]) + P - 1) // P)) for _ in range(Hkv)] for b in range(B)]
    lists, counts = _lists_from(sets, bt.shape[1])
    scale = 0.37
    out, lse = O.sparse_decode(q, kp, vp, bt, lens, P, lists, counts, Hkv, O.PER_KV_HEAD, scale)
    for b in range(B):
        L = int(lens[b])
        for h in range(Hq):
            g = h // G
            eo, el = sdpa(q[b, :, h], K[b, g, :L], V[b, g, :L], scale, np.ones((T, L), bool))
            assert np.allclose(out[b, :, h], eo, atol=1e-12, rtol=1e-10), (b, h)
            assert np.allclose(lse[b, :, h], el, atol=1e-12, rtol=1e-10), (b, h)


def check_decode_masked_sdpa():
    """Page-list attention == dense attention with unselected tokens masked (per q head)."""
    rng = np.random.default_rng(7)
    q, K, V, kp, vp, bt, lens = _dense_decode_case(rng, Hq=6, Hkv=2, lens=(23, 17))
    B, T, Hq, _ = q.shape
    Hkv, P = 2, 4
    G = Hq // Hkv
    sets = []
    for b in range(B):
        n = (int(lens[b]) + P - 1) // P
        sets.append([set(int(x) for x in rng.choice(n, size=int(rng.integers(1, n + 1)), replace=False))
                     for _ in range(Hq)])
    lists, counts = _lists_from(sets, bt.shape[1])
    scale = 0.5
    out, lse = O.sparse_decode(q, kp, vp, bt, lens, P, lists, counts, Hkv, O.PER_Q_HEAD, scale)
    for b in range(B):
        L = int(lens[b])
        for h in range(Hq):
            allowed = np.array([(j // P) in sets[b][h] for j in range(L)])[None, :].repeat(T, 0)
            eo, el = sdpa(q[b, :, h], K[b, h // G, :L], V[b, h // G, :L], scale, allowed)
            assert np.allclose(out[b, :, h], eo, atol=1e-12, rtol=1e-10), (b, h)
            assert np.allclose(lse[b, :, h], el, atol=1e-12, rtol=1e-10), (b, h)


def check_decode_golden():
    with open(os.path.join(GOLDEN, "decode_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        kp = np.array(c["k_pool"], dtype=np.float64)
        vp = np.array(c["v_pool"], dtype=np.float64)
        bt = np.array([c["block_table"]], dtype=np.int32)
        q = np.array(c["q"], dtype=np.float64)[None, None, None, :]
        lst = np.array([[c["list"] + [-1] * (bt.shape[1] - len(c["list"]))]], dtype=np.int32)
        cnt = np.array([[len(c["list"])]], dtype=np.int32)
        out, lse = O.sparse_decode(q, kp, vp, bt, np.array([c["seq_len"]]), c["page_size"], lst, cnt,
                                   1, O.PER_KV_HEAD, c["sm_scale"])
        assert np.allclose(out[0, 0, 0], c["o"], atol=1e-12), (c["name"], out[0, 0, 0])
        assert abs(lse[0, 0, 0] - c["lse"]) < 1e-12, (c["name"], lse[0, 0, 0])


def check_decode_closed_forms():
    rng = np.random.default_rng(8)
    q, K, V, kp, vp, bt, lens = _dense_decode_case(rng, B=1, T=1, Hq=2, Hkv=1, lens=(13,))
    P = 4
    # V = const  ->  o = const for any selection
    Vc = np.full_like(V, 2.5)
    kpc, vpc, btc = scatter_to_pool(K, Vc, P, rng)
    lists, counts = _lists_from([[{0, 2, 3}]], btc.shape[1])
    out, _ = O.sparse_decode(q, kpc, vpc, btc, lens, P, lists, counts, 1, O.PER_KV_HEAD, 0.3)
    assert np.allclose(out, 2.5, atol=1e-13)
    # single valid token (last page holds 1 token of 13) -> o = V_j, lse = z_j
    lists, counts = _lists_from([[{3}]], bt.shape[1])
    out, lse = O.sparse_decode(q, kp, vp, bt, lens, P, lists, counts, 1, O.PER_KV_HEAD, 0.3)
    for h in range(2):
        assert np.allclose(out[0, 0, h], V[0, 0, 12], atol=1e-13)
        assert abs(lse[0, 0, h] - 0.3 * float(q[0, 0, h] @ K[0, 0, 12])) < 1e-12
    # one-hot V rows -> o is the softmax weight vector: non-negative, sums to 1
    L = 13
    Vid = np.eye(L)[None, None]
    kpi, vpi, bti = scatter_to_pool(K, Vid, P, rng)
    lists, counts = _lists_from([[{0, 1, 2, 3}]], bti.shape[1])
    out, _ = O.sparse_decode(q, kpi, vpi, bti, lens, P, lists, counts, 1, O.PER_KV_HEAD, 0.3, d_v=L)
    w = out[0, 0]
    assert (w >= 0).all() and np.allclose(w.sum(axis=-1), 1.0, atol=1e-14)
    # empty list -> o = 0, lse = -inf
    lists, counts = _lists_from([[set()]], bt.shape[1])
    out, lse = O.sparse_decode(q, kp, vp, bt, lens, P, lists, counts, 1, O.PER_KV_HEAD, 0.3)
    assert (out == 0).all() and np.isneginf(lse).all()


def check_decode_large_logits():
    rng = np.random.default_rng(9)
    q, K, V, kp, vp, bt, lens = _dense_decode_case(rng, B=1, T=1, Hq=2, Hkv=1, lens=(16,))
    P = 4
    scale = 300.0            # logits in the thousands: exp overflows without the max shift
    lists, counts = _lists_from([[{0, 1, 2, 3}]], bt.shape[1])
    out, lse = O.sparse_decode(q, kp, vp, bt, lens, P, lists, counts, 1, O.PER_KV_HEAD, scale)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    for h in range(2):
        eo, el = sdpa(q[0, :, h], K[0, 0], V[0, 0], scale, np.ones((1, 16), bool))
        assert np.allclose(out[0, :, h], eo, atol=1e-9) and np.allclose(lse[0, :, h], el, rtol=1e-12)


def check_decode_pool_permutation():
    """The physical placement of pages never changes the result (bit-identical)."""
    rng = np.random.default_rng(10)
    q, K, V, kp, vp, bt, lens = _dense_decode_case(rng)
    kp2, vp2, bt2 = scatter_to_pool(K, V, 4, np.random.default_rng(99), extra_pages=7)
    sets = [[{0, 2, 4}, {1, 3}], [{0, 1}, {2}]]
    lists, counts = _lists_from(sets, bt.shape[1])
    a = O.sparse_decode(q, kp, vp, bt, lens, 4, lists, counts, 2, O.PER_KV_HEAD, 0.4)
    b = O.sparse_decode(q, kp2, vp2, bt2, lens, 4, lists, counts, 2, O.PER_KV_HEAD, 0.4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def check_decode_modes_and_tiers():
    rng = np.random.default_rng(11)
    q, K, V, kp, vp, bt, lens = _dense_decode_case(rng, Hq=4, Hkv=2, lens=(29, 21))
    B, T, Hq, _ = q.shape
    Hkv, P, G = 2, 4, 2
    sets = [[{0, 3, 5}, {1, 2}], [{0, 4}, {5}]]
    lists, counts = _lists_from(sets, bt.shape[1])
    grp = O.sparse_decode(q, kp, vp, bt, lens, P, lists, counts, Hkv, O.PER_KV_HEAD, 0.4)
    # per-q mode with each head given its group's list == group mode, bit for bit
    qsets = [[sets[b][h // G] for h in range(Hq)] for b in range(B)]
    ql, qc = _lists_from(qsets, bt.shape[1])
    per = O.sparse_decode(q, kp, vp, bt, lens, P, ql, qc, Hkv, O.PER_Q_HEAD, 0.4)
    assert np.array_equal(grp[0], per[0]) and np.array_equal(grp[1], per[1])
    # tiered: list = Critical (first 1 entry) + Ambient; every head in every mask == untiered
    cc = np.ones((B, Hkv), dtype=np.int32)
    all_heads = np.full((B, bt.shape[1], 1), (1 << Hq) - 1, dtype=np.int64)
    tier = O.sparse_decode(q, kp, vp, bt, lens, P, lists, counts, Hkv, O.PER_KV_HEAD, 0.4, cc, all_heads)
    assert np.array_equal(tier[0], grp[0])
    # no head in any Ambient mask == untiered over the Critical segment only
    none = np.zeros((B, bt.shape[1], 1), dtype=np.int64)
    tier0 = O.sparse_decode(q, kp, vp, bt, lens, P, lists, counts, Hkv, O.PER_KV_HEAD, 0.4, cc, none)
    crit = _lists_from([[{min(s)} for s in sets[b]] for b in range(B)], bt.shape[1])
    ref0 = O.sparse_decode(q, kp, vp, bt, lens, P, crit[0], crit[1], Hkv, O.PER_KV_HEAD, 0.4)
    assert np.array_equal(tier0[0], ref0[0])
    # mixed mask: head h sees Ambient page p iff bit h of p's mask -> masked SDPA per head
    mixed = rng.integers(0, 1 << Hq, size=(B, bt.shape[1], 1)).astype(np.int64)
    tm = O.sparse_decode(q, kp, vp, bt, lens, P, lists, counts, Hkv, O.PER_KV_HEAD, 0.4, cc, mixed)
    for b in range(B):
        L = int(lens[b])
        for h in range(Hq):
            s = h // G
            ordered = sorted(sets[b][s])
            seen = {ordered[0]} | {p for p in ordered[1:] if (int(mixed[b, p, 0]) >> h) & 1}
            allowed = np.array([(j // P) in seen for j in range(L)])[None, :].repeat(T, 0)
            eo, el = sdpa(q[b, :, h], K[b, s, :L], V[b, s, :L], 0.4, allowed)
            assert np.allclose(tm[0][b, :, h], eo, atol=1e-12) and np.allclose(tm[1][b, :, h], el, atol=1e-12)


def check_decode_split_merge():
    rng = np.random.default_rng(12)
    q, K, V, kp, vp, bt, lens = _dense_decode_case(rng, B=1, T=1, Hq=2, Hkv=1, lens=(40,))
    P = 4
    full = list(range(10))
    lists, counts = _lists_from([[set(full)]], bt.shape[1])
    ref_o, ref_l = O.sparse_decode(q, kp, vp, bt, lens, P, lists, counts, 1, O.PER_KV_HEAD, 0.3)
    for ns in (1, 2, 3, 4, 7, 10, 13):
        rngs = O.split_ranges(len(full), ns)
        assert [r for r in rngs if r[1] > r[0]][-1][1] == len(full)
        sizes = [e - s for s, e in rngs]
        assert max(sizes) - min(sizes) <= 1 and sum(sizes) == len(full)
        po, pl = [], []
        for (s0, s1) in rngs:
            sub = _lists_from([[set(full[s0:s1])]], bt.shape[1])
            o, l = O.sparse_decode(q, kp, vp, bt, lens, P, sub[0], sub[1], 1, O.PER_KV_HEAD, 0.3)
            po.append(o[0, 0])
            pl.append(l[0, 0])
        po, pl = np.stack(po, 1), np.stack(pl, 1)   # [Hq][S][dv], [Hq][S]
        for h in range(2):
            mo, ml = O.lse_merge(po[h], pl[h])
            assert np.allclose(mo, ref_o[0, 0, h], atol=1e-13, rtol=1e-12), ns
            assert abs(ml - ref_l[0, 0, h]) < 1e-12


def check_decode_latent_sdpa():
    """Latent cache (no V pool): V is the first d_v dims of each cached row, K the whole row.

    The rope tail of every row is large and distinct, so reading V from any other
    dims (or K from only the first d_v) moves the output far beyond the tolerance.
    Checked against torch float64 SDPA on explicitly built V = K[..., :d_v], for
    Critical-only lists and for tiered lists with a mixed Ambient head mask.
    """
    rng = np.random.default_rng(16)
    B, T, Hq, P, dl, dr = 2, 2, 4, 4, 8, 4
    d = dl + dr
    lens = (22, 15)
    L = max(lens)
    q = rng.standard_normal((B, T, Hq, d))
    K = rng.standard_normal((B, 1, L, d))
    K[..., dl:] = 5.0 + 3.0 * np.arange(dr) + rng.standard_normal((B, 1, L, dr))
    kp, _, bt = scatter_to_pool(K, K[..., :dl], P, rng, extra_pages=2)
    scale = 0.2
    sets = [[{0, 2, 5}], [{1, 3}]]
    lists, counts = _lists_from(sets, bt.shape[1])
    lens_a = np.array(lens)
    # Critical only: every head of the single latent head attends the whole list
    out, lse = O.sparse_decode(q, kp, None, bt, lens_a, P, lists, counts, 1, O.PER_KV_HEAD, scale, d_v=dl)
    assert out.shape == (B, T, Hq, dl)
    for b in range(B):
        Lb = lens[b]
        allowed = np.array([(j // P) in sets[b][0] for j in range(Lb)])[None, :].repeat(T, 0)
        Kd = K[b, 0, :Lb]
        Vd = np.array(Kd[:, :dl])
        for h in range(Hq):
            eo, el = sdpa(q[b, :, h], Kd, Vd, scale, allowed)
            assert np.allclose(out[b, :, h], eo, atol=1e-12, rtol=1e-10), (b, h)
            assert np.allclose(lse[b, :, h], el, atol=1e-12, rtol=1e-10), (b, h)
    # tiered: the first listed page is Critical, the rest Ambient under a mixed head mask
    cc = np.ones((B, 1), dtype=np.int32)
    mixed = rng.integers(0, 1 << Hq, size=(B, bt.shape[1], 1)).astype(np.int64)
    to, tl = O.sparse_decode(q, kp, None, bt, lens_a, P, lists, counts, 1, O.PER_KV_HEAD, scale, cc, mixed,
                             d_v=dl)
    for b in range(B):
        Lb = lens[b]
        ordered = sorted(sets[b][0])
        Kd = K[b, 0, :Lb]
        Vd = np.array(Kd[:, :dl])
        for h in range(Hq):
            seen = {ordered[0]} | {p for p in ordered[1:] if (int(mixed[b, p, 0]) >> h) & 1}
            allowed = np.array([(j // P) in seen for j in range(Lb)])[None, :].repeat(T, 0)
            eo, el = sdpa(q[b, :, h], Kd, Vd, scale, allowed)
            assert np.allclose(to[b, :, h], eo, atol=1e-12) and np.allclose(tl[b, :, h], el, atol=1e-12), (b, h)


# ------------------------------------------------------------------- a6-a7
def check_union_bruteforce():
    rng = np.random.default_rng(13)
    for trial in range(30):
        Hkv = int(rng.integers(1, 4))
        G = int(rng.integers(1, 4))
        Hq, nqb, nkb = Hkv * G, int(rng.integers(1, 5)), int(rng.integers(1, 30))
        mask = (rng.random((Hq, nqb, nkb)) < rng.random() * 0.3).astype(np.uint8)
        tables, counts = O.gqa_union_block_table(mask, Hkv)
        for g in range(Hkv):
            exp = set()
            for h in range(g * G, (g + 1) * G):
                for qb in range(nqb):
                    for kb in range(nkb):
                        if mask[h, qb, kb]:
                            exp.add(kb)
            got = [int(x) for x in tables[g, :counts[g]]]
            assert got == sorted(exp), (trial, g)
            assert (tables[g, counts[g]:] == -1).all()
    # group size 1 with one Q-block: the table is the mask row itself
    m = (rng.random((3, 1, 17)) < 0.4).astype(np.uint8)
    t, c = O.gqa_union_block_table(m, 3)
    for h in range(3):
        assert [int(x) for x in t[h, :c[h]]] == list(np.flatnonzero(m[h, 0]))


def check_union_golden():
    with open(os.path.join(GOLDEN, "union_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        t, n = O.gqa_union_block_table(np.array(c["mask"], dtype=np.uint8), c["n_kv_heads"])
        assert t.tolist() == c["tables"] and n.tolist() == c["counts"], c["name"]


def _prefill_case(rng, Hq=4, Hkv=2, P=4, d=8, q_len=9, q_start=13):
    L = q_start + q_len
    q = rng.standard_normal((q_len, Hq, d))
    K = rng.standard_normal((1, Hkv, L, d))
    V = rng.standard_normal((1, Hkv, L, d))
    kp, vp, bt = scatter_to_pool(K, V, P, rng, extra_pages=2)
    return q, K, V, kp, vp, bt, L


def check_prefill_causal_sdpa():
    """All-causal-blocks mask == dense causal attention at offset q_start."""
    rng = np.random.default_rng(14)
    q, K, V, kp, vp, bt, L = _prefill_case(rng)
    q_len, Hq, d = q.shape
    Hkv, P, q_start, G = 2, 4, 13, 2
    nkb = (L + P - 1) // P
    tables = np.tile(np.arange(nkb, dtype=np.int32), (Hkv, 1))
    counts = np.full(Hkv, nkb, dtype=np.int32)
    out, lse = O.block_sparse_prefill(q, kp, vp, bt[0], L, P, q_start, tables, counts, Hkv, 0.35)
    causal = np.arange(L)[None, :] <= (q_start + np.arange(q_len))[:, None]
    for h in range(Hq):
        eo, el = sdpa(q[:, h], K[0, h // G], V[0, h // G], 0.35, causal)
        assert np.allclose(out[:, h], eo, atol=1e-12) and np.allclose(lse[:, h], el, atol=1e-12), h
    # rows subset gives the same numbers
    sub = [(0, 1), (8, 3), (4, 0)]
    so, sl = O.block_sparse_prefill(q, kp, vp, bt[0], L, P, q_start, tables, counts, Hkv, 0.35, rows=sub)
    for (i, h) in sub:
        # (BLAS may order a different row count differently: last-bit agreement only)
        assert np.allclose(so[i, h], out[i, h], atol=1e-14, rtol=1e-12) and abs(sl[i, h] - lse[i, h]) < 1e-12


def check_prefill_masked_sdpa():
    """Random block mask: every query of a group sees exactly the group's union blocks, causally."""
    rng = np.random.default_rng(15)
    q, K, V, kp, vp, bt, L = _prefill_case(rng, Hq=6, Hkv=2, q_len=11, q_start=21)
    q_len, Hq, d = q.shape
    Hkv, P, q_start, G = 2, 4, 21, 3
    nkb = (L + P - 1) // P
    nqb = 3
    mask = (rng.random((Hq, nqb, nkb)) < 0.3).astype(np.uint8)
    tables, counts = O.gqa_union_block_table(mask, Hkv)
    out, lse = O.block_sparse_prefill(q, kp, vp, bt[0], L, P, q_start, tables, counts, Hkv, 0.35)
    for h in range(Hq):
        g = h // G
        blocks = set(int(x) for x in tables[g, :counts[g]])
        allowed = np.array([[(j // P) in blocks and j <= q_start + i for j in range(L)] for i in range(q_len)])
        eo, el = sdpa(q[:, h], K[0, g], V[0, g], 0.35, allowed)
        empty = ~allowed.any(axis=1)
        assert np.allclose(out[~empty, h], eo[~empty], atol=1e-12), h
        assert np.allclose(lse[~empty, h], el[~empty], atol=1e-12), h
        assert (out[empty, h] == 0).all() and np.isneginf(lse[empty, h]).all()


# ------------------------------------------------------------ prefill mask
def _brute_mask(q, K_dense, scale, P, q_start, bq, nkb, n_kv, seq_len, top_k, max_gap):
    """Pure-Python reference for the block mask on a dense per-group key array K_dense[g][L][d]."""
    q_len, Hq, d = q.shape
    G = Hq // n_kv
    nqb = (q_len + bq - 1) // bq
    out = np.zeros((Hq, nqb, nkb), dtype=np.uint8)
    n_seq = (seq_len + P - 1) // P
    for h in range(Hq):
        g = h // G
        for qb in range(nqb):
            rows = list(range(qb * bq, min((qb + 1) * bq, q_len)))
            qbar = [math.fsum(float(q[i, h, e]) for i in rows) / len(rows) for e in range(d)]
            last = q_start + rows[-1]
            n = min(last // P + 1, n_seq, nkb)
            kb_lo = min((q_start + rows[0]) // P, n - 1)
            sc = []
            for kb in range(n):
                toks = [j for j in range(kb * P, (kb + 1) * P) if j < seq_len]
                mean_k = [math.fsum(float(K_dense[g, j, e]) for j in toks) / len(toks) for e in range(d)]
                sc.append(float(np.float32(scale * math.fsum(qbar[e] * mean_k[e] for e in range(d)))))
            forced = set([0]) | set(range(kb_lo, n))
            cand = [kb for kb in range(n) if kb not in forced]
            if top_k is not None:
                chosen = sorted(cand, key=lambda kb: (-sc[kb], kb))[:min(top_k, len(cand))]
            else:
                thr = float(np.float32(np.float32(max(sc)) - np.float32(max_gap)))
                chosen = [kb for kb in cand if sc[kb] >= thr]
            for kb in forced | set(chosen):
                out[h, qb, kb] = 1
    return out


def _mask_case(rng, integer):
    Hq, Hkv, P, d, bq = 4, 2, 4, 6, 4
    q_len, q_start = 10, 13
    L = q_start + q_len
    if integer:
        q = rng.integers(-3, 4, size=(q_len, Hq, d)).astype(np.float64)
        K = rng.integers(-4, 5, size=(1, Hkv, L, d)).astype(np.float64)
    else:
        q = rng.standard_normal((q_len, Hq, d))
        K = rng.standard_normal((1, Hkv, L, d))
    kp, _, bt = scatter_to_pool(K, K, P, rng, extra_pages=2)
    mu = O.page_summary(kp, bt, np.array([L]), P)
    return q, K[0], kp, bt[0], mu, Hkv, P, bq, q_start, L


def check_mask_bruteforce():
    """Integer-valued inputs make every mean and score exact, so exact score
    ties occur and must go to the lowest block index; real-valued inputs check
    the threshold mode."""
    rng = np.random.default_rng(17)
    for trial in range(6):
        integer = trial % 2 == 0
        q, Kd, kp, bt, mu, Hkv, P, bq, q_start, L = _mask_case(rng, integer)
        nkb = (L + P - 1) // P
        scale = 0.5
        for mode in ({"top_k": 0}, {"top_k": 1}, {"top_k": 2}, {"top_k": 50}, {"max_gap": 0.0},
                     {"max_gap": 1.5}, {"max_gap": float("inf")}):
            got, sc = O.prefill_block_mask(q, mu, bt, L, P, q_start, bq, nkb, Hkv, scale, **mode)
            exp = _brute_mask(q, Kd, scale, P, q_start, bq, nkb, Hkv, L, mode.get("top_k"), mode.get("max_gap"))
            assert np.array_equal(got, exp), (trial, mode)


def check_mask_invariants():
    rng = np.random.default_rng(18)
    q, Kd, kp, bt, mu, Hkv, P, bq, q_start, L = _mask_case(rng, False)
    nkb = (L + P - 1) // P
    q_len, Hq, _ = q.shape
    nqb = (q_len + bq - 1) // bq
    none, _ = O.prefill_block_mask(q, mu, bt, L, P, q_start, bq, nkb, Hkv, 0.3, top_k=0)
    every, _ = O.prefill_block_mask(q, mu, bt, L, P, q_start, bq, nkb, Hkv, 0.3, top_k=10 ** 6)
    gap_inf, _ = O.prefill_block_mask(q, mu, bt, L, P, q_start, bq, nkb, Hkv, 0.3, max_gap=float("inf"))
    assert np.array_equal(every, gap_inf)
    for qb in range(nqb):
        first, last = q_start + qb * bq, q_start + min((qb + 1) * bq, q_len) - 1
        causal = np.zeros(nkb, dtype=np.uint8)
        causal[:last // P + 1] = 1
        forced = np.zeros(nkb, dtype=np.uint8)
        forced[0] = 1
        forced[first // P:last // P + 1] = 1
        for h in range(Hq):
            assert np.array_equal(none[h, qb], forced), (h, qb)      # top_k = 0: sink + diagonal only
            assert np.array_equal(every[h, qb], causal), (h, qb)     # everything causal, nothing beyond


def check_mask_union_keeps_selection():
    """The union block tables built from a produced mask keep every block it selects."""
    rng = np.random.default_rng(19)
    q, Kd, kp, bt, mu, Hkv, P, bq, q_start, L = _mask_case(rng, False)
    nkb = (L + P - 1) // P
    mask, _ = O.prefill_block_mask(q, mu, bt, L, P, q_start, bq, nkb, Hkv, 0.3, top_k=1)
    tables, counts = O.gqa_union_block_table(mask, Hkv)
    G = q.shape[1] // Hkv
    for h in range(q.shape[1]):
        kept = set(int(x) for x in tables[h // G, :counts[h // G]])
        assert set(np.flatnonzero(mask[h].any(axis=0)).tolist()) <= kept


# ------------------------------------------------------------------ FP8
def check_fp8_decoding():
    """Every E4M3 byte against torch's float8_e4m3fn (an independent
    implementation of the OCP format), plus hand-derived values."""
    codes = np.arange(256, dtype=np.uint8)
    got = O.fp8_e4m3_to_float(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan], ref[~nan])
    hand = {0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0x3C: 1.5, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9,
            0x07: 7 * 2.0 ** -9, 0xC0: -2.0, 0xB8: -1.0, 0x80: -0.0}
    for c, v in hand.items():
        assert got[c] == v and np.signbit(got[c]) == np.signbit(v), (hex(c), got[c], v)


def check_fp8_decode_sdpa():
    """Decode over FP8 pages with per-page scales: the oracle's dequantised
    pools give torch float64 SDPA on the dense values dequantised with torch's
    own FP8 conversion."""
    rng = np.random.default_rng(20)
    B, T, Hq, Hkv, P, d = 2, 1, 4, 2, 4, 8
    lens = (14, 9)
    L = max(lens)
    npg = (L + P - 1) // P
    n_phys = B * npg + 1
    kq = rng.integers(0, 256, size=(n_phys, Hkv, P, d)).astype(np.uint8)
    vq = rng.integers(0, 256, size=(n_phys, Hkv, d, P)).astype(np.uint8)
    kq[(kq & 0x7F) == 0x7F] = 0x30          # no NaN codes
    vq[(vq & 0x7F) == 0x7F] = 0x30
    ks = rng.uniform(0.001, 0.02, size=(n_phys, Hkv)).astype(np.float32)
    vs = rng.uniform(0.1, 2.0, size=(n_phys, Hkv)).astype(np.float32)
    perm = rng.permutation(n_phys)
    bt = np.full((B, npg), -1, dtype=np.int32)
    for b in range(B):
        bt[b] = perm[b * npg:(b + 1) * npg]
    q = rng.standard_normal((B, T, Hq, d))
    kd = O.dequantize_pages(kq, ks)
    vd = O.dequantize_pages(vq, vs)
    sets = [[{0, 2}, {1, 3}], [{0, 1, 2}, {2}]]
    lists, counts = _lists_from(sets, npg)
    out, lse = O.sparse_decode(q, kd, vd, bt, np.array(lens), P, lists, counts, Hkv, O.PER_KV_HEAD, 0.35)
    tk = torch.from_numpy(kq).view(torch.float8_e4m3fn).to(torch.float64).numpy() * ks[:, :, None, None]
    tv = torch.from_numpy(vq).view(torch.float8_e4m3fn).to(torch.float64).numpy() * vs[:, :, None, None]
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            g = h // G
            toks = [(lp, r) for lp in sorted(sets[b][g]) for r in range(P) if lp * P + r < lens[b]]
            K = np.stack([tk[bt[b, lp], g, r] for lp, r in toks])
            V = np.stack([tv[bt[b, lp], g, :, r] for lp, r in toks])
            eo, el = sdpa(q[b, :, h], K, V, 0.35, np.ones((T, len(toks)), bool))
            assert np.allclose(out[b, :, h], eo, atol=1e-12) and np.allclose(lse[b, :, h], el, atol=1e-12), (b, h)


# ------------------------------------------------------- mean correction
def check_value_summary_bruteforce():
    rng = np.random.default_rng(21)
    B, Hkv, P, dv = 2, 2, 4, 5
    lens = [11, 6]
    L = max(lens)
    V = rng.standard_normal((B, Hkv, L, dv))
    _, vp, bt = scatter_to_pool(V, V, P, rng)
    nu = O.page_value_summary(vp, bt, np.array(lens), P)
    for b in range(B):
        for lp in range((lens[b] + P - 1) // P):
            toks = [j for j in range(lp * P, (lp + 1) * P) if j < lens[b]]
            for g in range(Hkv):
                for e in range(dv):
                    exp = math.fsum(V[b, g, j, e] for j in toks) / len(toks)
                    assert abs(float(nu[bt[b, lp], g, e]) - exp) <= 1e-6 * max(1.0, abs(exp))


def check_mean_correction_exact_on_constant_blocks():
    """When every token of a block carries the block's one key and one value,
    a skipped block's n_b * exp(z_b) term is exactly its tokens' sum, so the
    corrected prefill equals dense causal attention (torch float64 SDPA); with
    a full table it equals the plain block-sparse prefill."""
    rng = np.random.default_rng(22)
    Hq, Hkv, P, d = 4, 2, 4, 6
    q_len, q_start = 7, 17
    L = q_start + q_len
    nkb = (L + P - 1) // P
    G = Hq // Hkv
    Kb = rng.standard_normal((1, Hkv, nkb, d))
    Vb = rng.standard_normal((1, Hkv, nkb, d))
    K = np.repeat(Kb, P, axis=2)[:, :, :L]
    V = np.repeat(Vb, P, axis=2)[:, :, :L]
    q = rng.standard_normal((q_len, Hq, d))
    kp, vp, bt = scatter_to_pool(K, V, P, rng, extra_pages=1)
    # keep block 0 and the chunk's blocks; skip the rest
    keep = sorted({0} | set(range(q_start // P, nkb)))
    tables = np.full((Hkv, nkb), -1, dtype=np.int32)
    tables[:, :len(keep)] = keep
    counts = np.full(Hkv, len(keep), dtype=np.int32)
    out, lse = O.mean_corrected_prefill(q, kp, vp, bt[0], L, P, q_start, tables, counts, Hkv, 0.4)
    causal = np.arange(L)[None, :] <= (q_start + np.arange(q_len))[:, None]
    for h in range(Hq):
        eo, el = sdpa(q[:, h], K[0, h // G], V[0, h // G], 0.4, causal)
        assert np.allclose(out[:, h], eo, atol=1e-12) and np.allclose(lse[:, h], el, atol=1e-12), h
    # nothing skipped: the plain block-sparse prefill
    full = np.tile(np.arange(nkb, dtype=np.int32), (Hkv, 1))
    fc = np.full(Hkv, nkb, dtype=np.int32)
    a = O.mean_corrected_prefill(q, kp, vp, bt[0], L, P, q_start, full, fc, Hkv, 0.4)
    b = O.block_sparse_prefill(q, kp, vp, bt[0], L, P, q_start, full, fc, Hkv, 0.4)
    assert np.allclose(a[0], b[0], atol=1e-12) and np.allclose(a[1], b[1], atol=1e-12)


def check_mean_correction_bruteforce():
    """Random keys: the corrected output against the formula written out with
    explicit sums (math.fsum) over the table's tokens and the skipped blocks'
    means; skipped blocks past a query's position (wholly or partly) add
    nothing."""
    rng = np.random.default_rng(23)
    Hq, Hkv, P, d = 2, 1, 4, 3
    q_len, q_start = 6, 13
    L = q_start + q_len
    nkb = (L + P - 1) // P
    K = rng.standard_normal((1, Hkv, L, d))
    V = rng.standard_normal((1, Hkv, L, d))
    q = rng.standard_normal((q_len, Hq, d))
    kp, vp, bt = scatter_to_pool(K, V, P, rng)
    keep = [1, 4]
    tables = np.full((Hkv, nkb), -1, dtype=np.int32)
    tables[0, :2] = keep
    counts = np.array([2], dtype=np.int32)
    out, lse = O.mean_corrected_prefill(q, kp, vp, bt[0], L, P, q_start, tables, counts, Hkv, 0.7)
    for i in range(q_len):
        pos = q_start + i
        for h in range(Hq):
            terms = []      # (log weight, value vector)
            for kb in range(nkb):
                toks = [j for j in range(kb * P, min((kb + 1) * P, L))]
                if kb in keep:
                    for j in toks:
                        if j <= pos:
                            terms.append((0.7 * math.fsum(q[i, h, e] * K[0, 0, j, e] for e in range(d)), V[0, 0, j]))
                elif toks[-1] <= pos:
                    mk = [math.fsum(K[0, 0, j, e] for j in toks) / len(toks) for e in range(d)]
                    mv = np.array([math.fsum(V[0, 0, j, e] for j in toks) / len(toks) for e in range(d)])
                    terms.append((0.7 * math.fsum(q[i, h, e] * mk[e] for e in range(d)) + math.log(len(toks)), mv))
            m = max(t[0] for t in terms)
            w = [math.exp(t[0] - m) for t in terms]
            den = math.fsum(w)
            exp_o = [math.fsum(w[k] * terms[k][1][e] for k in range(len(terms))) / den for e in range(d)]
            assert np.allclose(out[i, h], exp_o, atol=1e-12), (i, h)
            assert abs(lse[i, h] - (m + math.log(den))) < 1e-12


# ---------------------------------------------------------------- autotuner
def _mass_case(rng, constant_pages):
    """Latent-free GQA case: B=2 sequences (one with a partial last page),
    T=2 query tokens, 4 query heads over 2 KV heads, pages of 4 tokens."""
    B, T, Hq, Hkv, P, d = 2, 2, 4, 2, 4, 5
    lens = [14, 9]
    L = max(lens)
    n_max = (L + P - 1) // P
    if constant_pages:
        Kp = rng.standard_normal((B, Hkv, n_max, d))
        K = np.repeat(Kp, P, axis=2)[:, :, :L]
    else:
        K = rng.standard_normal((B, Hkv, L, d))
    q = rng.standard_normal((B, T, Hq, d))
    kp, _, bt = scatter_to_pool(K, K[..., :1], P, rng, extra_pages=2)
    if constant_pages:
        mu = kp[:, :, 0, :].copy()           # the page's one key, exactly
    else:
        mu = O.page_summary(kp, bt, np.array(lens), P)
    return q, K, kp, bt, mu, lens, P, Hkv


def check_head_mass_exact_on_constant_pages():
    """When every token of a page carries the page's one key, a page's
    estimated mass is exactly its tokens' share of the true softmax over the
    sequence's tokens (explicit exp sums, math.fsum), summed over the query
    tokens; a partial last page weighs its own token count."""
    rng = np.random.default_rng(31)
    q, K, kp, bt, mu, lens, P, Hkv = _mass_case(rng, constant_pages=True)
    B, T, Hq, d = q.shape
    G = Hq // Hkv
    M = O.head_page_mass(q, mu, bt, np.array(lens), P, Hkv, 0.6)
    for b in range(B):
        n = (lens[b] + P - 1) // P
        assert np.all(np.isnan(M[b, :, n:]))
        for h in range(Hq):
            for p in range(n):
                exp = 0.0
                for t in range(T):
                    z = [0.6 * math.fsum(q[b, t, h, e] * K[b, h // G, j, e] for e in range(d)) for j in range(lens[b])]
                    m = max(z)
                    w = [math.exp(x - m) for x in z]
                    exp += math.fsum(w[j] for j in range(p * P, min((p + 1) * P, lens[b]))) / math.fsum(w)
                assert abs(M[b, h, p] - exp) <= 1e-12, (b, h, p)


def check_head_mass_rows_sum():
    """Random keys: every head's masses sum to the number of query tokens."""
    rng = np.random.default_rng(32)
    q, K, kp, bt, mu, lens, P, Hkv = _mass_case(rng, constant_pages=False)
    M = O.head_page_mass(q, mu, bt, np.array(lens), P, Hkv, 0.6)
    for b in range(q.shape[0]):
        n = (lens[b] + P - 1) // P
        assert np.allclose(M[b, :, :n].sum(axis=1), q.shape[1], atol=1e-12)
        assert np.all(M[b, :, :n] > 0)


def _tier_case(rng):
    B, Hq, Hkv, T = 2, 8, 2, 2
    n_pages = [9, 7]
    max_pages = 10
    M = np.full((B, Hq, max_pages), np.nan)
    for b in range(B):
        raw = rng.random((Hq, n_pages[b])) ** 3
        M[b, :, :n_pages[b]] = T * raw / raw.sum(axis=1, keepdims=True)
    scores = np.full((B, Hkv, max_pages), np.nan, dtype=np.float32)
    for b in range(B):
        scores[b, :, :n_pages[b]] = rng.integers(-3, 4, size=(Hkv, n_pages[b])).astype(np.float32)
    P = 4
    seq_lens = np.array([n * P - 1 for n in n_pages])
    return M, scores, seq_lens, P, Hkv, T, n_pages


def check_tier_coverage_matches_pair_sets():
    """Coverage of each configuration against the mass on the exact (head,
    page) pairs the tiered decode computes: lists from select_pages with
    top_k = alpha + beta and critical_k = alpha, the Ambient mask from
    ambient_head_mask, each head's pages from row_pages, summed with
    math.fsum."""
    rng = np.random.default_rng(33)
    M, scores, seq_lens, P, Hkv, T, n_pages = _tier_case(rng)
    B, Hq, _ = M.shape
    G = Hq // Hkv
    alphas, hs, budget, sink, window = [0, 1, 2, 4], [1, 2, 4], 14, 1, 1
    cov, beta, best = O.tier_coverage(M, scores, seq_lens, P, Hkv, T, sink, window, budget, alphas, hs)
    for ia, a in enumerate(alphas):
        for ih, h in enumerate(hs):
            if a * G > budget:
                assert np.isnan(cov[ia, ih]) and beta[ia, ih] == -1
                continue
            bt = (budget - a * G) // h
            assert beta[ia, ih] == bt
            lists, counts, cc = O.select_pages(scores, n_pages, sink, window, a + bt, a)
            mask = O.ambient_head_mask(M, lists, counts, cc, Hkv, h)
            per = []
            for b in range(B):
                for g in range(Hkv):
                    tot = []
                    for x in range(g * G, (g + 1) * G):
                        for p in O.row_pages(b, g, x, lists, counts, cc, mask):
                            tot.append(M[b, x, p])
                    per.append(math.fsum(tot) / (T * G))
            assert abs(cov[ia, ih] - math.fsum(per) / len(per)) <= 1e-12, (a, h)
    feas = [(cov[i, j], i, j) for i in range(len(alphas)) for j in range(len(hs)) if not np.isnan(cov[i, j])]
    top = max(c for c, _, _ in feas)
    assert best == min((i, j) for c, i, j in feas if c == top)


def check_ambient_mask_bruteforce():
    """The Ambient heads of a page maximise the page's covered mass over every
    head subset of that size (itertools-free enumeration over bitmasks); among
    equal masses the lowest head indices win."""
    B, Hq, Hkv, max_pages = 1, 8, 2, 5
    G = Hq // Hkv
    # integer masses with ties
    M = np.array([[[3, 1, 2, 2, 0], [1, 1, 2, 0, 5], [3, 1, 0, 2, 5], [0, 1, 2, 2, 1],
                   [2, 2, 2, 2, 2], [1, 3, 0, 1, 0], [2, 3, 1, 0, 4], [2, 0, 1, 1, 4]]], dtype=np.float64)
    lists = np.array([[[0, 2, 3, 4, -1], [1, 4, 0, 2, 3]]], dtype=np.int32)
    counts = np.array([[4, 5]], dtype=np.int32)
    cc = np.array([[1, 2]], dtype=np.int32)
    for h in (1, 2, 3, 4):
        mask = O.ambient_head_mask(M, lists, counts, cc, Hkv, h)
        bits_set = {(p, x) for p in range(max_pages) for x in range(Hq) if (int(mask[0, p, 0]) >> x) & 1}
        want = set()
        for g in range(Hkv):
            heads = list(range(g * G, (g + 1) * G))
            for e in range(cc[0, g], counts[0, g]):
                p = int(lists[0, g, e])
                best = None
                for bits in range(1 << G):
                    sub = [heads[i] for i in range(G) if (bits >> i) & 1]
                    if len(sub) != h:
                        continue
                    key = (-sum(M[0, x, p] for x in sub), sorted(sub))
                    if best is None or key < best:
                        best = key
                want |= {(p, x) for x in best[1]}
        assert bits_set == want, (h, sorted(bits_set ^ want))


def check_tier_special_cases():
    """h = G reduces to key-only selection (all heads on the first alpha +
    beta ranked pages); a budget covering every page with every head gives
    coverage 1; equal coverages pick the first configuration."""
    rng = np.random.default_rng(34)
    M, scores, seq_lens, P, Hkv, T, n_pages = _tier_case(rng)
    B, Hq, _ = M.shape
    G = Hq // Hkv
    cov, beta, best = O.tier_coverage(M, scores, seq_lens, P, Hkv, T, 0, 0, 12, [0, 1, 3], [G])
    for ia, a in enumerate([0, 1, 3]):
        k = a + (12 - a * G) // G
        per = []
        for b in range(B):
            for g in range(Hkv):
                order = sorted(range(n_pages[b]), key=lambda p: (-float(scores[b, g, p]), p))
                per.append(math.fsum(M[b, x, p] for p in order[:k] for x in range(g * G, (g + 1) * G)) / (T * G))
        assert abs(cov[ia, 0] - math.fsum(per) / len(per)) <= 1e-12
    cov, _, _ = O.tier_coverage(M, scores, seq_lens, P, Hkv, T, 1, 1, 100 * G, [10], [1, G])
    assert np.allclose(cov, 1.0, atol=1e-12)
    # alpha 0 and 1 with h = G and budget 2G: both take the first two ranked pages
    cov, _, best = O.tier_coverage(M, scores, seq_lens, P, Hkv, T, 0, 0, 2 * G, [0, 1], [G])
    assert abs(cov[0, 0] - cov[1, 0]) <= 1e-15 and best == (0, 0)


ALL_CHECKS = [
    check_summary_constant_pages, check_summary_bruteforce,
    check_scores_exact_integers, check_scores_linearity_and_unfactored,
    check_select_bruteforce, check_select_golden,
    check_decode_select_all_sdpa, check_decode_masked_sdpa, check_decode_golden,
    check_decode_closed_forms, check_decode_large_logits, check_decode_pool_permutation,
    check_decode_modes_and_tiers, check_decode_split_merge, check_decode_latent_sdpa,
    check_union_bruteforce, check_union_golden,
    check_prefill_causal_sdpa, check_prefill_masked_sdpa,
    check_mask_bruteforce, check_mask_invariants, check_mask_union_keeps_selection,
    check_fp8_decoding, check_fp8_decode_sdpa,
    check_value_summary_bruteforce, check_mean_correction_exact_on_constant_blocks, check_mean_correction_bruteforce,
    check_head_mass_exact_on_constant_pages, check_head_mass_rows_sum, check_tier_coverage_matches_pair_sets,
    check_ambient_mask_bruteforce, check_tier_special_cases,
]
