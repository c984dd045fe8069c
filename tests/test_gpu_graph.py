"""The library's calls captured in a HIP graph give the same bits on every
replay as the eager calls, with unrelated eager work and synchronisations
between the replays (the benchmark replays captured steps)."""
import numpy as np
import pytest
import torch

import sparse_attention_long_page_amd as S
import workloads as W
from test_gpu_decode import MANY_LISTS, MODE, gpu_inputs, make_kv

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _step_fns(wl, inp):
    kv = make_kv(inp, wl)
    mode = MODE[wl.mode]
    stride = wl.list_stride
    mu = S.sa_page_summary(kv) if wl.scores == "summary" else None
    lists = torch.full((wl.batch, wl.n_sel, stride), -1, dtype=torch.int32, device=DEV)
    counts = torch.zeros((wl.batch, wl.n_sel), dtype=torch.int32, device=DEV)
    cc = torch.zeros_like(counts) if wl.tiered else None
    sel_ws = torch.empty(max(1, S.sa_select_pages_workspace_size(wl.batch, wl.n_sel, wl.max_pages)),
                         dtype=torch.uint8, device=DEV)
    dec_ws = torch.empty(max(1, S.sa_sparse_decode_workspace_size(kv, wl.q_tokens, wl.n_q_heads, stride, mode, 3)),
                         dtype=torch.uint8, device=DEV)
    out = torch.empty((wl.batch, wl.q_tokens, wl.n_q_heads, wl.d_v), dtype=inp["q"].dtype, device=DEV)
    lse = torch.empty((wl.batch, wl.q_tokens, wl.n_q_heads), dtype=torch.float32, device=DEV)

    def summary():
        S.sa_page_summary(kv, last_pages=1, out=mu)

    def select_and_decode():
        S.sa_select_pages(kv, n_q_heads=wl.n_q_heads, mode=mode, sink_pages=wl.sink_pages,
                          window_pages=wl.window_pages, top_k=wl.top_k, q=inp["q"] if mu is not None else None,
                          page_summary=mu, scores=inp["scores"], critical_k=wl.critical_k, list_stride=stride,
                          workspace=sel_ws, out=(lists, counts, cc))
        S.sa_sparse_decode(kv, inp["q"], lists, counts, mode=mode, sm_scale=wl.sm_scale, critical_counts=cc,
                           ambient_head_mask=inp["ambient_mask"], num_splits=3, out=out, out_lse=lse,
                           workspace=dec_ws)

    def step():
        if mu is not None:
            summary()
        select_and_decode()

    results = [lists, counts, out, lse] + ([cc] if cc is not None else [])
    step.parts = (summary, select_and_decode, mu)
    return step, results


@pytest.mark.parametrize("name", ["llama3_decode_small", "token_head_decode_small", "mla_tiered_decode_small"])
def test_graph_replays_match_eager(name):
    wl = W.SMALL[name]
    inp = gpu_inputs(W.make_decode_inputs(wl, "cpu", seed=41))
    step, results = _step_fns(wl, inp)
    step()
    torch.cuda.synchronize()
    eager = [r.clone() for r in results]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for r in results:                      # poison the outputs between replays
            r.fill_(-7)
        other = torch.randn(1 << 20, device=DEV).sum()   # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(other)
        _assert_same(results, eager, rep)


def _assert_same(results, eager, rep):
    """Lists are compared up to their counts (entries past a count are left
    untouched by the library); everything else element by element."""
    lists, counts = results[0], results[1]
    assert torch.equal(counts, eager[1]), f"replay {rep}: counts differ"
    L, E, C = lists.cpu().numpy(), eager[0].cpu().numpy(), counts.cpu().numpy()
    for idx in np.ndindex(*C.shape):
        n = int(C[idx])
        assert np.array_equal(L[idx][:n], E[idx][:n]), f"replay {rep}: list {idx} differs"
    for a, b in zip(results[2:], eager[2:]):
        assert torch.equal(a, b), f"replay {rep} differs from the eager result"


def test_prefill_graph_replays_match_eager():
    wl = W.SMALL["chunked_prefill_small"]
    inp = gpu_inputs(W.make_prefill_inputs(wl, "cpu", seed=42))
    kv = S.PagedKV(inp["k_pool"], inp["v_pool"], inp["block_table"], inp["seq_lens"])
    out = torch.empty((wl.q_len, wl.n_q_heads, wl.d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((wl.q_len, wl.n_q_heads), dtype=torch.float32, device=DEV)
    table = torch.full((wl.n_kv_heads, wl.n_kv_blocks), -1, dtype=torch.int32, device=DEV)
    counts = torch.zeros((wl.n_kv_heads,), dtype=torch.int32, device=DEV)

    def step():
        S.sa_block_sparse_prefill(kv, 0, inp["q"], wl.q_start, inp["block_mask"], wl.block_q, wl.sm_scale,
                                  out=out, out_lse=lse, block_table_out=table, block_counts_out=counts)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (out, lse, table, counts)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (out, lse, table, counts):
            t.fill_(-3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(counts, eager[3])
        for g_ in range(wl.n_kv_heads):
            n = int(counts[g_])
            assert torch.equal(table[g_, :n], eager[2][g_, :n]), f"replay {rep}: table {g_} differs"
        assert torch.equal(out, eager[0]) and torch.equal(lse, eager[1]), f"replay {rep} differs"


@pytest.mark.parametrize("name", ["llama3_decode_small", "llama3_many_lists"])
def test_summary_beside_selection_matches_serial(name):
    """With a local window the newest page is forced and its summary takes no
    part in the ranking; forced pages' summary rows take no part in the
    selection, so the newest-page summary update may run on a second stream beside
    the selection and the decode.  Graph replays of that forked step equal the
    serial eager step (fused score+select and separate kernels alike)."""
    wl = {**W.SMALL, **MANY_LISTS}[name]
    assert wl.window_pages >= 1 and wl.scores == "summary"
    inp = gpu_inputs(W.make_decode_inputs(wl, "cpu", seed=43))
    step, results = _step_fns(wl, inp)
    summary, select_and_decode, mu = step.parts
    step()
    torch.cuda.synchronize()
    eager = [r.clone() for r in results]
    side = torch.cuda.Stream()

    def forked():
        cur = torch.cuda.current_stream()
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            summary()
        select_and_decode()
        cur.wait_stream(side)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        forked()
    for rep in range(4):
        for r in results:
            r.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _assert_same(results, eager, rep)


@pytest.mark.parametrize("name", ["llama3_decode_small", "llama3_many_lists"])
def test_select_decode_graph_replays_match_eager(name):
    """The fused selection + decode call (newest-page summary recomputed inside)
    captured in a graph: every replay, with the outputs poisoned and unrelated
    eager work between replays, equals the eager call."""
    wl = {**W.SMALL, **MANY_LISTS}[name]
    inp = gpu_inputs(W.make_decode_inputs(wl, "cpu", seed=44))
    kv = make_kv(inp, wl)
    mu = S.sa_page_summary(kv)
    stride = wl.list_stride
    lists = torch.full((wl.batch, wl.n_sel, stride), -1, dtype=torch.int32, device=DEV)
    counts = torch.zeros((wl.batch, wl.n_sel), dtype=torch.int32, device=DEV)
    out = torch.empty((wl.batch, wl.q_tokens, wl.n_q_heads, wl.d_v), dtype=inp["q"].dtype, device=DEV)
    lse = torch.empty((wl.batch, wl.q_tokens, wl.n_q_heads), dtype=torch.float32, device=DEV)
    results = [lists, counts, out, lse]

    def step():
        S.sa_select_decode(kv, inp["q"], mu, sink_pages=wl.sink_pages, window_pages=wl.window_pages,
                           top_k=wl.top_k, sm_scale=wl.sm_scale, refresh_newest_page=True, list_stride=stride,
                           out=(lists, counts, out, lse))

    step()
    torch.cuda.synchronize()
    eager = [r.clone() for r in results]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for r in results:
            r.fill_(-7)
        other = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(other)
        _assert_same(results, eager, rep)


def test_prefill_mask_and_mean_correction_graph_replays_match_eager():
    """The block-sparse prefill chain captured in one graph: the mask from
    pattern discovery, the prefill over its union tables, the per-page value
    means and the mean correction (which rewrites out and lse in place).
    Every replay, with the outputs poisoned and eager work between replays,
    equals the eager chain."""
    wl = W.SMALL["chunked_prefill_small"].replace(random_fraction=0.15)
    inp = gpu_inputs(W.make_prefill_inputs(wl, "cpu", seed=45))
    kv = S.PagedKV(inp["k_pool"], inp["v_pool"], inp["block_table"], inp["seq_lens"])
    mu = S.sa_page_summary(kv)
    nu = S.sa_page_value_summary(kv)
    mask = torch.empty((wl.n_q_heads, wl.n_q_blocks, wl.n_kv_blocks), dtype=torch.uint8, device=DEV)
    out = torch.empty((wl.q_len, wl.n_q_heads, wl.d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((wl.q_len, wl.n_q_heads), dtype=torch.float32, device=DEV)
    table = torch.full((wl.n_kv_heads, wl.n_kv_blocks), -1, dtype=torch.int32, device=DEV)
    counts = torch.zeros((wl.n_kv_heads,), dtype=torch.int32, device=DEV)
    ws = torch.empty(S.sa_prefill_mean_correction_workspace_size(kv, wl.n_kv_blocks), dtype=torch.uint8, device=DEV)

    def step():
        S.sa_prefill_block_mask(kv, 0, inp["q"], wl.q_start, mu, wl.block_q, wl.sm_scale, top_k=2, out=mask)
        S.sa_page_value_summary(kv, out=nu)
        S.sa_block_sparse_prefill(kv, 0, inp["q"], wl.q_start, mask, wl.block_q, wl.sm_scale, out=out, out_lse=lse,
                                  block_table_out=table, block_counts_out=counts)
        S.sa_prefill_mean_correction(kv, 0, inp["q"], wl.q_start, table, counts, mu, nu, wl.sm_scale, out, lse,
                                     workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (mask, out, lse, counts, nu)]
    assert int(counts.min()) < wl.n_kv_blocks            # blocks are skipped, so the correction has work
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (mask, out, lse, counts):
            t.fill_(0)
        nu[nu == nu] = 0.0                             # the pages the chain rewrites
        other = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(other)
        for a, b in zip((mask, out, lse, counts), eager):
            assert torch.equal(a, b), f"replay {rep} differs from the eager chain"
        assert torch.equal(torch.nan_to_num(nu, nan=-1.0), torch.nan_to_num(eager[4], nan=-1.0))


def test_autotune_graph_replays_match_eager():
    """Head mass, tier search and Ambient head mask captured in one graph:
    every replay equals the eager calls (the mask is cleared by a kernel, not
    a memset node)."""
    wl = W.SMALL["mla_tiered_decode_small"]
    inp = gpu_inputs(W.make_decode_inputs(wl, "cpu", seed=46))
    kv = make_kv(inp, wl)
    mu = S.sa_page_summary(kv)
    G = wl.n_q_heads
    lists, counts, cc = S.sa_select_pages(kv, n_q_heads=G, mode=S.SA_SEL_PER_KV_HEAD, sink_pages=0, window_pages=0,
                                          top_k=wl.top_k, critical_k=wl.critical_k, q=inp["q"], page_summary=mu)
    scores = torch.empty((wl.batch, 1, wl.max_pages), dtype=torch.float32, device=DEV)
    S.sa_select_pages(kv, n_q_heads=G, mode=S.SA_SEL_PER_KV_HEAD, sink_pages=0, window_pages=0, top_k=wl.top_k,
                      q=inp["q"], page_summary=mu, scores_out=scores)
    mass = torch.empty((wl.batch, G, wl.max_pages), dtype=torch.float32, device=DEV)
    ws_m = torch.empty(S.sa_head_page_mass_workspace_size(kv, wl.q_tokens, G), dtype=torch.uint8, device=DEV)
    alphas, heads = [0, 1, 3], [4, 8, 32]
    ws_t = torch.empty(S.sa_autotune_tiers_workspace_size(kv, len(heads)), dtype=torch.uint8, device=DEV)
    cov = torch.empty((len(alphas), len(heads)), dtype=torch.float32, device=DEV)
    choice = torch.empty((3,), dtype=torch.int32, device=DEV)
    amask = torch.empty((wl.batch, wl.max_pages, (G + 31) // 32), dtype=torch.int32, device=DEV)
    budget = wl.critical_k * G + (wl.top_k - wl.critical_k) * wl.ambient_heads

    def step():
        S.sa_head_page_mass(kv, inp["q"], mu, wl.sm_scale, out=mass, workspace=ws_m)
        S.sa_autotune_tiers(kv, mass, scores, q_tokens=wl.q_tokens, sink_pages=0, window_pages=0, budget=budget,
                            alphas=alphas, ambient_heads=heads, workspace=ws_t, out=(cov, choice))
        S.sa_ambient_head_mask(kv, mass, lists, counts, cc, wl.ambient_heads, out=amask)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (mass, cov, choice, amask)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (mass, cov, choice, amask):
            t.fill_(-5)
        other = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(other)
        m_now, m_ref = mass.clone(), eager[0].clone()
        for b in range(wl.batch):                    # entries past a sequence's pages are not written
            n = (int(inp["seq_lens"][b]) + wl.page_size - 1) // wl.page_size
            m_now[b, :, n:] = 0
            m_ref[b, :, n:] = 0
        assert torch.equal(m_now, m_ref), f"replay {rep}: mass differs"
        for a, b in zip((cov, choice, amask), eager[1:]):
            assert torch.equal(a, b), f"replay {rep} differs from the eager calls"
