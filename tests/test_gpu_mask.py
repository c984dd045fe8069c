"""HIP block-mask producer (pooled-query block scores, top-k or max-gap
threshold) against the oracle, through the C ABI.  Masks must equal the
oracle's except inside the 1e-4 tie band around a row's selection threshold
(the k-th candidate score in top-k mode, max - max_gap in threshold mode);
the sink and diagonal blocks are always set and no block past a Q-block's
last position ever is."""
import math

import numpy as np
import pytest
import torch

import oracle.sparse_attn_oracle as O
import sparse_attention_long_page_amd as S
import workloads as W
from _parity import TIE_BAND, np64, npi

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _check_rows(got, exp, scores, mode, q_len, q_start, bq, P, band=TIE_BAND):
    """Returns the number of rows that differ from the oracle (tolerated band events)."""
    Hq, nqb, nkb = exp.shape
    events = 0
    for h in range(Hq):
        for qb in range(nqb):
            g, e = got[h, qb], exp[h, qb]
            if np.array_equal(g, e):
                continue
            events += 1
            first = q_start + qb * bq
            last = q_start + min((qb + 1) * bq, q_len) - 1
            n = int(np.count_nonzero(~np.isnan(scores[h, qb])))
            assert n == last // P + 1 or n < last // P + 1
            assert not g[n:].any(), (h, qb, "block past the causal range")
            kb_lo = min(first // P, n - 1)
            forced = {0} | set(range(kb_lo, n))
            assert all(g[kb] == 1 for kb in forced), (h, qb, "forced block missing")
            cand = [kb for kb in range(n) if kb not in forced]
            sc = scores[h, qb]
            chosen = {kb for kb in cand if g[kb]}
            if "top_k" in mode:
                k = min(mode["top_k"], len(cand))
                assert len(chosen) == k, (h, qb, len(chosen), k)
                ranked = O.rank_candidates(sc, cand)
                thr = float(sc[ranked[k - 1]]) if k else math.inf
            else:
                thr = float(np.float32(np.float32(np.nanmax(sc[:n])) - np.float32(mode["max_gap"])))
            for kb in cand:
                v = float(sc[kb])
                if v > thr + band:
                    assert kb in chosen, (h, qb, kb, v, thr)
                if v < thr - band:
                    assert kb not in chosen, (h, qb, kb, v, thr)
    return events


MODES = [{"top_k": 0}, {"top_k": 3}, {"top_k": 9}, {"top_k": 10 ** 4}, {"max_gap": 0.0}, {"max_gap": 0.4},
         {"max_gap": 2.0}, {"max_gap": float("inf")}]
SMALL = W.SMALL["chunked_prefill_small"]
CASES = {
    # ragged query tail (200 = 3*64 + 8), chunk start inside a page, group 4
    "g4": SMALL,
    # group 8 at the start of the sequence, and group 1 with a chunk shorter than a Q-block
    "g8_start": SMALL.replace(n_q_heads=8, n_kv_heads=1, q_len=150, q_start=0),
    "g1_short": SMALL.replace(n_q_heads=2, n_kv_heads=2, q_len=40, q_start=777),
}


@pytest.mark.parametrize("mode", MODES, ids=[str(m) for m in MODES])
@pytest.mark.parametrize("name", list(CASES))
def test_block_mask_matches_oracle(name, mode):
    wl = CASES[name]
    cpu = W.make_prefill_inputs(wl, "cpu", seed=71)
    inp = {k: v.to(DEV) for k, v in cpu.items()}
    kv = S.PagedKV(inp["k_pool"], inp["v_pool"], inp["block_table"], inp["seq_lens"])
    mu = S.sa_page_summary(kv)
    scale = float(np.float32(wl.sm_scale))
    got = S.sa_prefill_block_mask(kv, 0, inp["q"], wl.q_start, mu, wl.block_q, scale, n_kv_blocks=wl.n_kv_blocks,
                                  **mode)
    torch.cuda.synchronize()
    exp, sc = O.prefill_block_mask(np64(cpu["q"]), mu.cpu().numpy(), npi(cpu["block_table"])[0],
                                   int(cpu["seq_lens"][0]), wl.page_size, wl.q_start, wl.block_q, wl.n_kv_blocks,
                                   wl.n_kv_heads, scale, **mode)
    events = _check_rows(npi(got), exp, sc, mode, wl.q_len, wl.q_start, wl.block_q, wl.page_size)
    assert events <= 2, f"{events} rows differ"


def test_block_mask_feeds_the_union_and_prefill():
    """The produced mask goes straight into sa_block_sparse_prefill: tables
    bit-exact against the oracle's union of the same mask."""
    wl = SMALL
    cpu = W.make_prefill_inputs(wl, "cpu", seed=72)
    inp = {k: v.to(DEV) for k, v in cpu.items()}
    kv = S.PagedKV(inp["k_pool"], inp["v_pool"], inp["block_table"], inp["seq_lens"])
    mu = S.sa_page_summary(kv)
    mask = S.sa_prefill_block_mask(kv, 0, inp["q"], wl.q_start, mu, wl.block_q, wl.sm_scale, top_k=2,
                                   n_kv_blocks=wl.n_kv_blocks)
    out, lse, table, counts = S.sa_block_sparse_prefill(kv, 0, inp["q"], wl.q_start, mask, wl.block_q, wl.sm_scale)
    torch.cuda.synchronize()
    o_tab, o_cnt = O.gqa_union_block_table(npi(mask), wl.n_kv_heads)
    assert np.array_equal(npi(counts), o_cnt)
    for g in range(wl.n_kv_heads):
        assert np.array_equal(npi(table)[g, :o_cnt[g]], o_tab[g, :o_cnt[g]])


def test_full_size_block_mask_first_and_last_q_block():
    """The 128K chunk (32/8 heads, 2048 queries at 126976, 2016 KV blocks),
    top-160 per row (~8% of the causal blocks): every head's first and last
    Q-block row against the oracle."""
    wl = W.CHUNKED_PREFILL_128K
    inp = W.make_prefill_inputs(wl, DEV, seed=73)
    kv = S.PagedKV(inp["k_pool"], inp["v_pool"], inp["block_table"], inp["seq_lens"])
    mu = S.sa_page_summary(kv)
    scale = float(np.float32(wl.sm_scale))
    mode = {"top_k": 160}
    got = npi(S.sa_prefill_block_mask(kv, 0, inp["q"], wl.q_start, mu, wl.block_q, scale,
                                      n_kv_blocks=wl.n_kv_blocks, **mode))
    torch.cuda.synchronize()
    q = np64(inp["q"])
    mu_h = mu.cpu().numpy()
    bt = npi(inp["block_table"])[0]
    L = int(inp["seq_lens"][0])
    events = 0
    for qb in (0, wl.n_q_blocks - 1):
        i0, i1 = qb * wl.block_q, min((qb + 1) * wl.block_q, wl.q_len)
        exp, sc = O.prefill_block_mask(q[i0:i1], mu_h, bt, L, wl.page_size, wl.q_start + i0, wl.block_q,
                                       wl.n_kv_blocks, wl.n_kv_heads, scale, **mode)
        events += _check_rows(got[:, qb:qb + 1], exp, sc, mode, i1 - i0, wl.q_start + i0, wl.block_q,
                              wl.page_size)
    assert events <= 4, f"{events} rows differ"
