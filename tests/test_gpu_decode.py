"""HIP decode path (page summary, router scores, selection, split-K decode,
LSE merge) against the CPU oracle, through the C ABI."""
import math

import numpy as np
import pytest
import torch

import oracle.sparse_attn_oracle as O
import sparse_attention_long_page_amd as S
import workloads as W
from _parity import check_page_lists, compare_outputs, np64, npi, oracle_pools, sub_pool

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MODE = {"per_kv_head": S.SA_SEL_PER_KV_HEAD, "per_q_head": S.SA_SEL_PER_Q_HEAD}
DECODE_SMALL = [n for n, w in W.SMALL.items() if isinstance(w, W.DecodeWorkload) and not w.latent]


def gpu_inputs(cpu):
    return {k: (v.to(DEV) if v is not None else None) for k, v in cpu.items()}


def make_kv(inp, wl):
    return S.PagedKV(inp["k_pool"], inp["v_pool"], inp["block_table"], inp["seq_lens"], d_v=wl.d_v,
                     k_scale=inp.get("k_scale"), v_scale=inp.get("v_scale"))


def oracle_chain(cpu, wl):
    """Oracle mean keys, scores and lists from the CPU copy of the inputs."""
    bt, lens = npi(cpu["block_table"]), npi(cpu["seq_lens"])
    npg = [O.n_pages_of(L, wl.page_size) for L in lens]
    mu = scores = None
    if wl.scores == "gumbel":
        scores = npi(cpu["scores"])
    else:
        mu = O.page_summary(oracle_pools(cpu)[0], bt, lens, wl.page_size)
        scores = O.page_scores(np64(cpu["q"]), mu, bt, lens, wl.page_size, wl.n_kv_heads, wl.mode)
    lists, counts, cc = O.select_pages(scores, npg, wl.sink_pages, wl.window_pages, wl.top_k, wl.critical_k)
    return mu, scores, lists, counts, cc, npg


def gpu_select(inp, wl, kv, mu=None):
    if wl.scores == "gumbel":
        return S.sa_select_pages(kv, n_q_heads=wl.n_q_heads, mode=MODE[wl.mode], sink_pages=wl.sink_pages,
                                 window_pages=wl.window_pages, top_k=wl.top_k, scores=inp["scores"],
                                 critical_k=wl.critical_k), None
    scores_out = torch.empty((wl.batch, wl.n_sel, wl.max_pages), dtype=torch.float32, device=DEV)
    res = S.sa_select_pages(kv, n_q_heads=wl.n_q_heads, mode=MODE[wl.mode], sink_pages=wl.sink_pages,
                            window_pages=wl.window_pages, top_k=wl.top_k, q=inp["q"], page_summary=mu,
                            critical_k=wl.critical_k, scores_out=scores_out)
    return res, scores_out


@pytest.mark.parametrize("name", [n for n in DECODE_SMALL if W.SMALL[n].scores == "summary"])
def test_page_summary_matches_oracle(name):
    wl = W.SMALL[name]
    cpu = W.make_decode_inputs(wl, "cpu", seed=1)
    inp = gpu_inputs(cpu)
    mu_gpu = S.sa_page_summary(make_kv(inp, wl))
    torch.cuda.synchronize()
    mu_ref = O.page_summary(oracle_pools(cpu)[0], npi(cpu["block_table"]), npi(cpu["seq_lens"]), wl.page_size)
    got = mu_gpu.cpu().numpy()
    ref_pages = ~np.isnan(mu_ref[:, 0, 0])
    assert np.isnan(got[~ref_pages]).all(), "pages outside every sequence must stay untouched"
    diff = np.abs(got[ref_pages].astype(np.float64) - mu_ref[ref_pages])
    ulp = np.spacing(np.abs(mu_ref[ref_pages]).astype(np.float32)).astype(np.float64)
    assert (diff <= ulp).all(), f"max diff {diff.max()}"
    # incremental update of the last page only touches those pages
    mu2 = torch.full_like(mu_gpu, float("nan"))
    S.sa_page_summary(make_kv(inp, wl), last_pages=1, out=mu2)
    torch.cuda.synchronize()
    m2 = mu2.cpu().numpy()
    bt, lens = npi(cpu["block_table"]), npi(cpu["seq_lens"])
    last = {int(bt[b, O.n_pages_of(L, wl.page_size) - 1]) for b, L in enumerate(lens)}
    touched = {int(p) for p in np.flatnonzero(~np.isnan(m2[:, 0, 0]))}
    assert touched == last
    for p in last:
        assert np.array_equal(m2[p], got[p])


# enough lists (batch x selection heads >= 128) for the fused score+select kernel
MANY_LISTS = {
    "llama3_many_lists": W.SMALL["llama3_decode_small"].replace(
        name="llama3_many_lists", batch=17, n_q_heads=32, n_kv_heads=8,
        seq_lens=tuple(64 * (9 + 3 * i) + (i * 13) % 64 for i in range(17))),
    # 128 lists (one workgroup each scores and selects) over sequences with no
    # page, one page, only forced pages and a single candidate
    "short_many_lists": W.SMALL["llama3_decode_small"].replace(
        name="short_many_lists", batch=16, n_q_heads=32, n_kv_heads=8,
        seq_lens=(0, 1, 64, 65, 64 * 3, 64 * 3 + 5, 64 * 9 + 1, 64 * 20, 0, 2, 63, 128, 129, 64 * 4, 64 * 5 + 3, 7)),
    "per_q_summary_many_lists": W.SMALL["token_head_decode_small"].replace(
        name="per_q_summary_many_lists", batch=4, n_q_heads=32, n_kv_heads=8, scores="summary",
        context=16 * 90 + 7, top_k=12, sink_pages=1, window_pages=3, num_splits=2),
}
# the one-workgroup-per-list scoring kernel at the other head dims and dtypes
MANY_LISTS.update({
    "bf16_d64_many_lists": W.SMALL["bf16_d64_p16_kv_small"].replace(
        name="bf16_d64_many_lists", batch=32, n_q_heads=16, n_kv_heads=4,
        seq_lens=tuple(16 * (5 + 7 * i) + (i * 5) % 16 for i in range(32))),
    "fp32_d64_many_lists": W.SMALL["fp32_d64_p16_q_small"].replace(
        name="fp32_d64_many_lists", batch=32, seq_lens=tuple(16 * (4 + 3 * i) + i % 16 for i in range(32))),
    "fp32_d128_many_lists": W.SMALL["fp32_d128_p64_kv_small"].replace(
        name="fp32_d128_many_lists", batch=64, n_q_heads=8, n_kv_heads=2,
        seq_lens=tuple(64 * (4 + i % 13) + (i * 11) % 64 for i in range(64))),
    # 128 sequences over one latent head: 576-d scores, tiered lists
    "latent_many_lists": W.SMALL["mla_tiered_decode_small"].replace(
        name="latent_many_lists", batch=128, n_q_heads=16, ambient_heads=4, context=0, top_k=4, critical_k=2,
        seq_lens=tuple(64 * (1 + i % 9) + (i * 7) % 64 for i in range(128))),
})
SELECT_CASES = {**{n: W.SMALL[n] for n in DECODE_SMALL}, **MANY_LISTS}


@pytest.mark.parametrize("name", list(SELECT_CASES))
def test_select_matches_oracle(name):
    wl = SELECT_CASES[name]
    cpu = W.make_decode_inputs(wl, "cpu", seed=2)
    inp = gpu_inputs(cpu)
    kv = make_kv(inp, wl)
    mu = S.sa_page_summary(kv) if wl.scores == "summary" else None
    (lists, counts, cc), scores_out = gpu_select(inp, wl, kv, mu)
    torch.cuda.synchronize()
    _, o_scores, o_lists, o_counts, o_cc, npg = oracle_chain(cpu, wl)
    if scores_out is not None:
        g = scores_out.cpu().numpy()
        assert np.array_equal(np.isnan(g), np.isnan(o_scores))
        fin = ~np.isnan(g)
        rel = np.abs(g[fin].astype(np.float64) - o_scores[fin]) / np.maximum(1.0, np.abs(o_scores[fin]))
        assert rel.max() <= 1e-6, rel.max()
    rep = check_page_lists(npi(lists), npi(counts), None if cc is None else npi(cc), o_scores, npg,
                           wl.sink_pages, wl.window_pages, wl.top_k, wl.critical_k)
    assert not rep.failures, rep.failures[:5]
    assert rep.exact + rep.band_events == rep.units


@pytest.mark.parametrize("name", [n for n, w in SELECT_CASES.items() if w.scores == "summary" and w.dtype != "fp8"])
def test_select_with_summary_refresh_matches_separate_calls(name):
    """refresh_newest_page: the selection first rewrites each sequence's
    newest-page summary (fused into the score+select kernel when there are
    enough lists, a separate summary kernel otherwise).  Its summaries, scores
    and lists equal those of sa_page_summary(last_pages=1) followed by a plain
    selection, bit for bit; the newest pages' rows start out poisoned, so the
    refresh must have written them."""
    wl = SELECT_CASES[name]
    cpu = W.make_decode_inputs(wl, "cpu", seed=5)
    inp = gpu_inputs(cpu)
    kv = make_kv(inp, wl)
    mu_ref = S.sa_page_summary(kv)
    bt, lens = npi(cpu["block_table"]), npi(cpu["seq_lens"])
    newest = [int(bt[b, O.n_pages_of(int(L), wl.page_size) - 1]) for b, L in enumerate(lens) if L > 0]
    mu_ref[newest] = float("nan")
    mu_fused = mu_ref.clone()
    args = dict(n_q_heads=wl.n_q_heads, mode=MODE[wl.mode], sink_pages=wl.sink_pages, window_pages=wl.window_pages,
                top_k=wl.top_k, q=inp["q"], critical_k=wl.critical_k)
    sc_ref = torch.empty((wl.batch, wl.n_sel, wl.max_pages), dtype=torch.float32, device=DEV)
    sc_fused = torch.empty_like(sc_ref)
    S.sa_page_summary(kv, last_pages=1, out=mu_ref)
    l_ref, c_ref, cc_ref = S.sa_select_pages(kv, page_summary=mu_ref, scores_out=sc_ref, **args)
    l_f, c_f, cc_f = S.sa_select_pages(kv, page_summary=mu_fused, scores_out=sc_fused, refresh_newest_page=True, **args)
    torch.cuda.synchronize()
    assert torch.equal(mu_fused.isnan(), mu_ref.isnan())
    assert torch.equal(torch.nan_to_num(mu_fused, nan=0.0), torch.nan_to_num(mu_ref, nan=0.0))
    assert not mu_ref[newest].isnan().any()
    assert torch.equal(torch.nan_to_num(sc_fused, nan=0.0), torch.nan_to_num(sc_ref, nan=0.0))
    assert torch.equal(c_f, c_ref)
    if cc_ref is not None:
        assert torch.equal(cc_f, cc_ref)
    L1, L2, C = npi(l_f), npi(l_ref), npi(c_ref)
    for idx in np.ndindex(*C.shape):
        assert np.array_equal(L1[idx][:C[idx]], L2[idx][:C[idx]]), idx


@pytest.mark.parametrize("tiered", [False, True])
def test_select_long_lists_with_ties_exact(tiered):
    """Selection on given scores is index work: it must equal the oracle's
    lists exactly.  Lists of up to 9000 pages (several pages per thread of the
    select workgroup), scores drawn from a few values (two of them adjacent
    floats) plus NaN and both zeros, so the threshold key has thousands of
    ties that must go to the lowest page indices."""
    P, max_pages, H = 16, 9000, 3
    lens = np.array([P * 9000, P * 5000 + 3, P * 513, P * 40 + 1], dtype=np.int32)
    B = len(lens)
    rng = np.random.default_rng(77)
    vals = np.array([-1.5, -0.0, 0.0, 0.25, np.nextafter(np.float32(0.25), np.float32(1)), 2.0, np.nan],
                    dtype=np.float32)
    scores = vals[rng.integers(0, len(vals), size=(B, H, max_pages))]
    sink, window, top_k = 2, 5, 2500
    crit = 700 if tiered else None
    kv = S.PagedKV(torch.zeros((4, 1, P, 64), dtype=torch.bfloat16, device=DEV),
                   torch.zeros((4, 1, 64, P), dtype=torch.bfloat16, device=DEV),
                   torch.zeros((B, max_pages), dtype=torch.int32, device=DEV), torch.from_numpy(lens).to(DEV))
    lists, counts, cc = S.sa_select_pages(kv, n_q_heads=H, mode=S.SA_SEL_PER_Q_HEAD, sink_pages=sink,
                                          window_pages=window, top_k=top_k,
                                          scores=torch.from_numpy(scores).to(DEV), critical_k=crit)
    torch.cuda.synchronize()
    npg = [O.n_pages_of(int(L), P) for L in lens]
    o_lists, o_counts, o_cc = O.select_pages(scores, npg, sink, window, top_k, crit)
    g_lists, g_counts = npi(lists), npi(counts)
    assert np.array_equal(g_counts, o_counts)
    if tiered:
        assert np.array_equal(npi(cc), o_cc)
    for b in range(B):
        for h in range(H):
            n = int(o_counts[b, h])
            assert np.array_equal(g_lists[b, h, :n], o_lists[b, h, :n]), (b, h)


# list lengths (pages) on both sides of each selection-kernel width: keys in
# registers for 1, 2 or 4 pages per thread (up to 512, 1024, 2048 pages), an
# LDS radix select beyond
PATH_EDGES = [1, 9, 64, 65, 511, 512, 513, 1024, 1025, 2047, 2048, 2049, 2600]


@pytest.mark.parametrize("top_k,crit", [(41, None), (41, 8), (700, None), (700, 300), (0, None)])
def test_select_list_sizes_across_paths_exact(top_k, crit):
    """Given scores, every list length around the kernel's width switches must
    give the oracle's lists exactly (4,096 and 8,192 pages: 8 and 16 keys per
    thread, read in 16-byte groups).  Head 0 draws from a few tied values (two
    adjacent floats, NaN, both zeros), head 1 from a normal distribution."""
    P, H = 16, 2
    edges = PATH_EDGES + [4096, 8192]
    lens = np.array([P * n - (n % 5) for n in edges], dtype=np.int32)
    B, max_pages = len(lens), max(edges)
    rng = np.random.default_rng(91)
    vals = np.array([-1.5, -0.0, 0.0, 0.25, np.nextafter(np.float32(0.25), np.float32(1)), 2.0, np.nan],
                    dtype=np.float32)
    scores = np.empty((B, H, max_pages), dtype=np.float32)
    scores[:, 0] = vals[rng.integers(0, len(vals), size=(B, max_pages))]
    scores[:, 1] = rng.standard_normal((B, max_pages)).astype(np.float32)
    sink, window = 1, 8
    kv = S.PagedKV(torch.zeros((4, 1, P, 64), dtype=torch.bfloat16, device=DEV),
                   torch.zeros((4, 1, 64, P), dtype=torch.bfloat16, device=DEV),
                   torch.zeros((B, max_pages), dtype=torch.int32, device=DEV), torch.from_numpy(lens).to(DEV))
    lists, counts, cc = S.sa_select_pages(kv, n_q_heads=H, mode=S.SA_SEL_PER_Q_HEAD, sink_pages=sink,
                                          window_pages=window, top_k=top_k,
                                          scores=torch.from_numpy(scores).to(DEV), critical_k=crit)
    torch.cuda.synchronize()
    npg = [O.n_pages_of(int(L), P) for L in lens]
    assert npg == edges
    o_lists, o_counts, o_cc = O.select_pages(scores, npg, sink, window, top_k, crit)
    g_lists, g_counts = npi(lists), npi(counts)
    assert np.array_equal(g_counts, o_counts)
    if crit is not None:
        assert np.array_equal(npi(cc), o_cc)
    for b in range(B):
        for h in range(H):
            n = int(o_counts[b, h])
            assert np.array_equal(g_lists[b, h, :n], o_lists[b, h, :n]), (npg[b], h)


# (KV heads, group size, query tokens): 128 lists scored and selected one
# workgroup each; 16 lists scored over blocks of pages whose last workgroup
# selects, with the pooled query summed inline (4 rows) or by the prep kernel
# in row chunks (64 rows)
LONG_LIST_SHAPES = [(8, 4, 1), (1, 4, 1), (1, 32, 2)]


@pytest.mark.parametrize("crit", [None, 8])
@pytest.mark.parametrize("shape", LONG_LIST_SHAPES, ids=["128_lists", "16_lists", "16_lists_pooled"])
def test_score_select_long_lists(crit, shape):
    """Router scores and selection on lists of up to 2600 pages, covering each
    selection width.  The page summaries are given (random fp32 rows), so the
    oracle needs no key pool.  Lists follow the tie-band rule against the
    oracle's scores; the scores written out agree to 1e-6 relative, and the
    same call without scores written out gives the same lists."""
    Hkv, G, T = shape
    P, d = 16, 128
    npg = PATH_EDGES[2:] + [40] * 5
    B, max_pages = len(npg), max(npg)
    lens = np.array([P * n - 3 for n in npg], dtype=np.int32)
    n_phys = sum(npg) + 7
    rng = np.random.default_rng(17)
    bt = np.zeros((B, max_pages), dtype=np.int32)
    perm = rng.permutation(n_phys).astype(np.int32)
    off = 0
    for b, n in enumerate(npg):
        bt[b, :n] = perm[off:off + n]
        off += n
    mu = rng.standard_normal((n_phys, Hkv, d)).astype(np.float32)
    q = torch.from_numpy(rng.standard_normal((B, T, Hkv * G, d)).astype(np.float32)).to(torch.bfloat16)
    kv = S.PagedKV(torch.empty((n_phys, Hkv, P, d), dtype=torch.bfloat16, device=DEV),
                   torch.empty((n_phys, Hkv, d, P), dtype=torch.bfloat16, device=DEV),
                   torch.from_numpy(bt).to(DEV), torch.from_numpy(lens).to(DEV))
    sink, window, top_k = 1, 8, 41
    scores_out = torch.empty((B, Hkv, max_pages), dtype=torch.float32, device=DEV)
    lists, counts, cc = S.sa_select_pages(kv, n_q_heads=Hkv * G, mode=S.SA_SEL_PER_KV_HEAD, sink_pages=sink,
                                          window_pages=window, top_k=top_k, q=q.to(DEV),
                                          page_summary=torch.from_numpy(mu).to(DEV), critical_k=crit,
                                          scores_out=scores_out)
    # the same selection without scores written out (the forced pages' rows are then not read)
    l2, c2, cc2 = S.sa_select_pages(kv, n_q_heads=Hkv * G, mode=S.SA_SEL_PER_KV_HEAD, sink_pages=sink,
                                    window_pages=window, top_k=top_k, q=q.to(DEV),
                                    page_summary=torch.from_numpy(mu).to(DEV), critical_k=crit)
    torch.cuda.synchronize()
    o_scores = O.page_scores(q.float().numpy().astype(np.float64), mu, bt, lens, P, Hkv, "per_kv_head")
    g = scores_out.cpu().numpy()
    assert np.array_equal(np.isnan(g), np.isnan(o_scores))
    fin = ~np.isnan(g)
    rel = np.abs(g[fin].astype(np.float64) - o_scores[fin]) / np.maximum(1.0, np.abs(o_scores[fin]))
    assert rel.max() <= 1e-6, rel.max()
    rep = check_page_lists(npi(lists), npi(counts), None if cc is None else npi(cc), o_scores, npg,
                           sink, window, top_k, crit)
    assert not rep.failures, rep.failures[:5]
    assert rep.exact + rep.band_events == rep.units
    assert torch.equal(c2, counts)
    C, L1, L2 = npi(counts), npi(lists), npi(l2)
    for idx in np.ndindex(*C.shape):
        assert np.array_equal(L1[idx][:C[idx]], L2[idx][:C[idx]]), idx


@pytest.mark.parametrize("name", DECODE_SMALL)
@pytest.mark.parametrize("splits", [1, 2, 3, 0])
def test_decode_matches_oracle(name, splits):
    wl = W.SMALL[name]
    cpu = W.make_decode_inputs(wl, "cpu", seed=3)
    inp = gpu_inputs(cpu)
    kv = make_kv(inp, wl)
    _, _, o_lists, o_counts, o_cc, _ = oracle_chain(cpu, wl)
    lists = torch.from_numpy(o_lists).to(DEV)
    counts = torch.from_numpy(o_counts).to(DEV)
    out, lse = S.sa_sparse_decode(kv, inp["q"], lists, counts, mode=MODE[wl.mode], sm_scale=wl.sm_scale,
                                  num_splits=splits)
    torch.cuda.synchronize()
    ref_o, ref_l = O.sparse_decode(np64(cpu["q"]), *oracle_pools(cpu),
                                   npi(cpu["block_table"]), npi(cpu["seq_lens"]), wl.page_size, o_lists,
                                   o_counts, wl.n_kv_heads, wl.mode, wl.sm_scale)
    compare_outputs(out, lse, ref_o, ref_l, fp32=wl.dtype == "fp32")


@pytest.mark.parametrize("name", ["llama3_decode_small", "token_head_decode_small"])
def test_tiered_small_heads_matches_oracle(name):
    """Critical/Ambient tiers on the d-128 kernel: Ambient pages only for masked heads."""
    base = W.SMALL[name]
    wl = base.replace(critical_k=2, ambient_heads=max(1, base.n_q_heads // 3))
    cpu = W.make_decode_inputs(wl, "cpu", seed=4)
    inp = gpu_inputs(cpu)
    kv = make_kv(inp, wl)
    _, o_scores, o_lists, o_counts, o_cc, npg = oracle_chain(cpu, wl)
    mu = S.sa_page_summary(kv) if wl.scores == "summary" else None
    (lists, counts, cc), _ = gpu_select(inp, wl, kv, mu)
    torch.cuda.synchronize()
    rep = check_page_lists(npi(lists), npi(counts), npi(cc), o_scores, npg, wl.sink_pages, wl.window_pages,
                           wl.top_k, wl.critical_k)
    assert not rep.failures, rep.failures[:5]
    amask = inp["ambient_mask"]
    out, lse = S.sa_sparse_decode(kv, inp["q"], torch.from_numpy(o_lists).to(DEV),
                                  torch.from_numpy(o_counts).to(DEV), mode=MODE[wl.mode], sm_scale=wl.sm_scale,
                                  critical_counts=torch.from_numpy(o_cc).to(DEV), ambient_head_mask=amask,
                                  num_splits=2)
    torch.cuda.synchronize()
    ref_o, ref_l = O.sparse_decode(np64(cpu["q"]), *oracle_pools(cpu),
                                   npi(cpu["block_table"]), npi(cpu["seq_lens"]), wl.page_size, o_lists,
                                   o_counts, wl.n_kv_heads, wl.mode, wl.sm_scale, o_cc,
                                   npi(cpu["ambient_mask"]).astype(np.int64) & 0xffffffff)
    compare_outputs(out, lse, ref_o, ref_l)


def test_decode_deterministic_and_pool_permutation_invariant():
    wl = W.SMALL["llama3_decode_small"]
    cpu = W.make_decode_inputs(wl, "cpu", seed=5)
    inp = gpu_inputs(cpu)
    kv = make_kv(inp, wl)
    _, _, o_lists, o_counts, _, _ = oracle_chain(cpu, wl)
    lists, counts = torch.from_numpy(o_lists).to(DEV), torch.from_numpy(o_counts).to(DEV)
    a = S.sa_sparse_decode(kv, inp["q"], lists, counts, mode=0, sm_scale=wl.sm_scale, num_splits=3)
    b = S.sa_sparse_decode(kv, inp["q"], lists, counts, mode=0, sm_scale=wl.sm_scale, num_splits=3)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    # move every page to another physical slot; same logical content -> same bits
    n_phys = inp["k_pool"].shape[0]
    perm = torch.randperm(n_phys, generator=torch.Generator().manual_seed(7)).to(DEV)
    k2 = torch.empty_like(inp["k_pool"]); k2[perm] = inp["k_pool"]
    v2 = torch.empty_like(inp["v_pool"]); v2[perm] = inp["v_pool"]
    bt = inp["block_table"]
    bt2 = torch.where(bt >= 0, perm[bt.clamp(min=0).long()].to(torch.int32), bt)
    kv2 = S.PagedKV(k2, v2, bt2.contiguous(), inp["seq_lens"])
    c = S.sa_sparse_decode(kv2, inp["q"], lists, counts, mode=0, sm_scale=wl.sm_scale, num_splits=3)
    torch.cuda.synchronize()
    assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1])


def test_empty_lists_and_streaming_mode():
    wl = W.SMALL["llama3_decode_small"].replace(top_k=0)
    cpu = W.make_decode_inputs(wl, "cpu", seed=6)
    inp = gpu_inputs(cpu)
    kv = make_kv(inp, wl)
    mu = S.sa_page_summary(kv)
    (lists, counts, _), _ = gpu_select(inp, wl, kv, mu)
    torch.cuda.synchronize()
    npg = [O.n_pages_of(L, wl.page_size) for L in wl.lengths()]
    for b in range(wl.batch):
        exp = O.forced_pages(npg[b], wl.sink_pages, wl.window_pages)
        for s in range(wl.n_sel):
            assert npi(lists)[b, s, :npi(counts)[b, s]].tolist() == exp
    # empty lists: o = 0, lse = -inf
    zeros = torch.zeros_like(counts)
    out, lse = S.sa_sparse_decode(kv, inp["q"], lists, zeros, mode=0, sm_scale=wl.sm_scale, num_splits=2)
    torch.cuda.synchronize()
    assert (out.float() == 0).all() and torch.isneginf(lse).all()


def _full_size_check(wl, seed, n_sample):
    """Full-size inputs on the GPU; the oracle checks a seeded sample of sequences."""
    inp = W.make_decode_inputs(wl, DEV, seed=seed)
    kv = make_kv(inp, wl)
    mu = S.sa_page_summary(kv) if wl.scores == "summary" else None
    (lists, counts, cc), scores_out = gpu_select(inp, wl, kv, mu)
    out, lse = S.sa_sparse_decode(kv, inp["q"], lists, counts, mode=MODE[wl.mode], sm_scale=wl.sm_scale,
                                  num_splits=wl.num_splits,
                                  critical_counts=cc, ambient_head_mask=inp["ambient_mask"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    picks = sorted(rng.choice(wl.batch, size=min(n_sample, wl.batch), replace=False).tolist())
    kp, vp, bt, lens = sub_pool(inp, picks)
    npg = [O.n_pages_of(L, wl.page_size) for L in lens]
    if wl.scores == "gumbel":
        o_scores = npi(inp["scores"])[picks]
    else:
        o_mu = O.page_summary(kp, bt, lens, wl.page_size)
        o_scores = O.page_scores(np64(inp["q"])[picks], o_mu, bt, lens, wl.page_size, wl.n_kv_heads, wl.mode)
    g_lists, g_counts = npi(lists)[picks], npi(counts)[picks]
    g_cc = None if cc is None else npi(cc)[picks]
    rep = check_page_lists(g_lists, g_counts, g_cc, o_scores, npg, wl.sink_pages, wl.window_pages, wl.top_k,
                           wl.critical_k)
    assert not rep.failures, rep.failures[:5]
    # attention: the oracle runs on the GPU's own (accepted) lists, so a tolerated
    # tie swap is never counted as an attention error and every row is compared
    amask = None if inp["ambient_mask"] is None else npi(inp["ambient_mask"])[picks].astype(np.int64) & 0xffffffff
    ref_o, ref_l = O.sparse_decode(np64(inp["q"])[picks], kp, vp, bt, lens, wl.page_size, g_lists, g_counts,
                                   wl.n_kv_heads, wl.mode, wl.sm_scale, g_cc, amask, d_v=wl.d_v)
    return compare_outputs(out[picks], lse[picks], ref_o, ref_l), rep


def test_full_size_llama3_decode_32k_sampled():
    (mx, mean, lse_err), rep = _full_size_check(W.LLAMA3_DECODE_32K, seed=11, n_sample=4)
    print(f"max_abs {mx:.3e} mean_abs {mean:.3e} lse {lse_err:.3e} band events {rep.band_events}/{rep.units}")


def test_full_size_llama3_decode_32k_fp8_sampled():
    """The Llama-3 32K layer over FP8 pages with per-page scales."""
    (mx, mean, lse_err), rep = _full_size_check(W.LLAMA3_DECODE_32K_FP8, seed=17, n_sample=4)
    print(f"max_abs {mx:.3e} mean_abs {mean:.3e} lse {lse_err:.3e} band events {rep.band_events}/{rep.units}")


def test_full_size_token_head_decode_128k_sampled():
    (mx, mean, lse_err), rep = _full_size_check(W.TOKEN_HEAD_DECODE_128K, seed=12, n_sample=2)
    print(f"max_abs {mx:.3e} mean_abs {mean:.3e} lse {lse_err:.3e} band events {rep.band_events}/{rep.units}")


def _select_then_decode(kv, inp, wl, mu, refresh):
    """The two calls sa_select_decode stands for (one decode split)."""
    lists, counts, _ = S.sa_select_pages(kv, n_q_heads=wl.n_q_heads, mode=S.SA_SEL_PER_KV_HEAD,
                                         sink_pages=wl.sink_pages, window_pages=wl.window_pages, top_k=wl.top_k,
                                         q=inp["q"], page_summary=mu, refresh_newest_page=refresh)
    out, lse = S.sa_sparse_decode(kv, inp["q"], lists, counts, mode=S.SA_SEL_PER_KV_HEAD, sm_scale=wl.sm_scale,
                                  num_splits=1)
    return lists, counts, out, lse


def _assert_same_step(a, b):
    (l1, c1, o1, s1), (l2, c2, o2, s2) = a, b
    assert torch.equal(c1, c2)
    L1, L2, C = npi(l1), npi(l2), npi(c1)
    for idx in np.ndindex(*C.shape):
        assert np.array_equal(L1[idx][:C[idx]], L2[idx][:C[idx]]), idx
    assert torch.equal(o1, o2)
    assert torch.equal(s1, s2)


@pytest.mark.parametrize("refresh", [False, True])
@pytest.mark.parametrize("name", ["llama3_decode_small", "llama3_many_lists"])
def test_select_decode_equals_select_then_decode(name, refresh):
    """sa_select_decode writes exactly what sa_select_pages followed by a
    one-split sa_sparse_decode write: lists, counts, output and lse bit for bit
    (and, with refresh, the newest pages' summaries); the small case is also
    checked against the oracle."""
    wl = SELECT_CASES[name]
    cpu = W.make_decode_inputs(wl, "cpu", seed=13)
    inp = gpu_inputs(cpu)
    kv = make_kv(inp, wl)
    mu_a = S.sa_page_summary(kv)
    mu_b = mu_a.clone()
    ref = _select_then_decode(kv, inp, wl, mu_a, refresh)
    got = S.sa_select_decode(kv, inp["q"], mu_b, sink_pages=wl.sink_pages, window_pages=wl.window_pages,
                             top_k=wl.top_k, sm_scale=wl.sm_scale, refresh_newest_page=refresh)
    torch.cuda.synchronize()
    _assert_same_step(got, ref)
    assert torch.equal(torch.nan_to_num(mu_a, nan=0.0), torch.nan_to_num(mu_b, nan=0.0))
    if name == "llama3_decode_small":
        _, o_scores, o_lists, o_counts, _, npg = oracle_chain(cpu, wl)
        rep = check_page_lists(npi(got[0]), npi(got[1]), None, o_scores, npg, wl.sink_pages, wl.window_pages,
                               wl.top_k, None)
        assert not rep.failures, rep.failures[:5]
        assert rep.exact == rep.units
        ref_o, ref_l = O.sparse_decode(np64(cpu["q"]), *oracle_pools(cpu),
                                       npi(cpu["block_table"]), npi(cpu["seq_lens"]), wl.page_size, o_lists,
                                       o_counts, wl.n_kv_heads, wl.mode, wl.sm_scale)
        compare_outputs(got[2], got[3], ref_o, ref_l)


def test_full_size_llama3_select_decode_equals_two_calls():
    """At the Llama-3 32K shape, in the decode step's form (newest-page refresh)."""
    wl = W.LLAMA3_DECODE_32K
    inp = W.make_decode_inputs(wl, DEV, seed=14)
    kv = make_kv(inp, wl)
    mu_a = S.sa_page_summary(kv)
    mu_b = mu_a.clone()
    ref = _select_then_decode(kv, inp, wl, mu_a, True)
    got = S.sa_select_decode(kv, inp["q"], mu_b, sink_pages=wl.sink_pages, window_pages=wl.window_pages,
                             top_k=wl.top_k, sm_scale=wl.sm_scale, refresh_newest_page=True)
    torch.cuda.synchronize()
    _assert_same_step(got, ref)
    assert torch.equal(mu_a, mu_b)


# empty sequence, one page (1 and 64 tokens), two pages, every page forced
# (3 pages = sink 1 + window 2), one candidate past the forced pages, 10 pages
SHORT_LENS = (0, 1, 64, 65, 64 * 3, 64 * 3 + 5, 64 * 9 + 1)


@pytest.mark.parametrize("refresh", [False, True])
def test_select_decode_short_and_empty_sequences(refresh):
    """Sequences with no page, one page, only forced pages, or one candidate:
    the fused call writes exactly what the two calls write, and the oracle's
    lists and attention (an empty sequence: empty list, o = 0, lse = -inf)."""
    wl = W.SMALL["llama3_decode_small"].replace(batch=len(SHORT_LENS), seq_lens=SHORT_LENS)
    cpu = W.make_decode_inputs(wl, "cpu", seed=21)
    inp = gpu_inputs(cpu)
    kv = make_kv(inp, wl)
    mu_a = S.sa_page_summary(kv)
    mu_b = mu_a.clone()
    ref = _select_then_decode(kv, inp, wl, mu_a, refresh)
    got = S.sa_select_decode(kv, inp["q"], mu_b, sink_pages=wl.sink_pages, window_pages=wl.window_pages,
                             top_k=wl.top_k, sm_scale=wl.sm_scale, refresh_newest_page=refresh)
    torch.cuda.synchronize()
    _assert_same_step(got, ref)
    assert torch.equal(torch.nan_to_num(mu_a, nan=0.0), torch.nan_to_num(mu_b, nan=0.0))
    _, o_scores, o_lists, o_counts, _, npg = oracle_chain(cpu, wl)
    assert npg == [0, 1, 1, 2, 3, 4, 10]
    g_lists, g_counts = npi(got[0]), npi(got[1])
    assert np.array_equal(g_counts, o_counts)
    for b in range(wl.batch):
        for s in range(wl.n_sel):
            assert np.array_equal(g_lists[b, s, :g_counts[b, s]], o_lists[b, s, :o_counts[b, s]]), (b, s)
    ref_o, ref_l = O.sparse_decode(np64(cpu["q"]), *oracle_pools(cpu),
                                   npi(cpu["block_table"]), npi(cpu["seq_lens"]), wl.page_size, o_lists,
                                   o_counts, wl.n_kv_heads, wl.mode, wl.sm_scale)
    compare_outputs(got[2], got[3], ref_o, ref_l)
    assert (got[2][0].float() == 0).all() and torch.isneginf(got[3][0]).all()


def test_select_decode_128k_context_equals_two_calls():
    """A 128K context (2,048 pages per list) through the fused call: the keys
    and the list fit the LDS beside the staging areas, and the result equals
    the two calls bit for bit, with the newest-page refresh."""
    wl = W.LLAMA3_DECODE_32K.replace(name="llama3_decode_128k_two", batch=2, context=131072)
    inp = W.make_decode_inputs(wl, DEV, seed=15)
    kv = make_kv(inp, wl)
    assert kv.max_pages >= 2048
    mu_a = S.sa_page_summary(kv)
    mu_b = mu_a.clone()
    ref = _select_then_decode(kv, inp, wl, mu_a, True)
    got = S.sa_select_decode(kv, inp["q"], mu_b, sink_pages=wl.sink_pages, window_pages=wl.window_pages,
                             top_k=wl.top_k, sm_scale=wl.sm_scale, refresh_newest_page=True)
    torch.cuda.synchronize()
    _assert_same_step(got, ref)
    assert torch.equal(mu_a, mu_b)


def test_select_decode_rejects_lists_beyond_lds():
    """max_pages + list_stride past what the LDS holds beside the staging
    areas: the call fails with SA_ERR_UNSUPPORTED and launches nothing."""
    wl = W.SMALL["llama3_decode_small"]
    inp = gpu_inputs(W.make_decode_inputs(wl, "cpu", seed=16))
    bt = torch.zeros((wl.batch, 8192), dtype=torch.int32, device=DEV)
    bt[:, :inp["block_table"].shape[1]] = inp["block_table"]
    kv = S.PagedKV(inp["k_pool"], inp["v_pool"], bt, inp["seq_lens"])
    mu = S.sa_page_summary(kv)
    with pytest.raises(S.SparseAttnError) as e:
        S.sa_select_decode(kv, inp["q"], mu, sink_pages=wl.sink_pages, window_pages=wl.window_pages,
                           top_k=wl.top_k, sm_scale=wl.sm_scale)
    assert e.value.status == S.SA_ERR_UNSUPPORTED and "LDS" in str(e.value)
