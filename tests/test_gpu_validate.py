"""Debug validation (sa_set_debug_validate): device-side checks of the index
data each call trusts.  Invalid entries planted from the host make the call
return SA_ERR_DATA naming the entry, with no output written; valid data gives
the same results, bit for bit, as with validation off.  Every kernel here
reads only in-range memory: the checks read the arrays within their declared
shapes, and the main kernels do not run on invalid data."""
import numpy as np
import pytest
import torch

import oracle.sparse_attn_oracle as O
import sparse_attention_long_page_amd as S
import workloads as W
from _parity import npi

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture
def validating():
    prev = S.sa_set_debug_validate(True)
    try:
        yield
    finally:
        S.sa_set_debug_validate(prev)


def _decode_case(name="llama3_decode_small", seed=61):
    wl = W.SMALL[name]
    cpu = W.make_decode_inputs(wl, "cpu", seed=seed)
    inp = {k: (v.to(DEV) if v is not None else None) for k, v in cpu.items()}
    bt, lens = npi(cpu["block_table"]), npi(cpu["seq_lens"])
    npg = [O.n_pages_of(L, wl.page_size) for L in lens]
    mu = O.page_summary(npi(cpu["k_pool"].float()).astype(np.float64), bt, lens, wl.page_size)
    sc = O.page_scores(npi(cpu["q"].float()).astype(np.float64), mu, bt, lens, wl.page_size, wl.n_kv_heads,
                       wl.mode)
    lists, counts, cc = O.select_pages(sc, npg, wl.sink_pages, wl.window_pages, wl.top_k, wl.critical_k)
    return wl, inp, lists, counts, cc, npg


def _kv(inp, wl, **over):
    t = dict(k_pool=inp["k_pool"], v_pool=inp["v_pool"], block_table=inp["block_table"],
             seq_lens=inp["seq_lens"])
    t.update(over)
    return S.PagedKV(t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"], d_v=wl.d_v)


def _expect_data_error(fn, needle):
    with pytest.raises(S.SparseAttnError) as e:
        fn()
    assert e.value.status == S.SA_ERR_DATA, str(e.value)
    assert needle in str(e.value), str(e.value)


def test_valid_data_same_results(validating):
    wl, inp, lists, counts, _, _ = _decode_case()
    kv = _kv(inp, wl)
    gl, gc = torch.from_numpy(lists).to(DEV), torch.from_numpy(counts).to(DEV)
    a = S.sa_sparse_decode(kv, inp["q"], gl, gc, mode=S.SA_SEL_PER_KV_HEAD, sm_scale=wl.sm_scale, num_splits=3)
    S.sa_set_debug_validate(False)
    b = S.sa_sparse_decode(kv, inp["q"], gl, gc, mode=S.SA_SEL_PER_KV_HEAD, sm_scale=wl.sm_scale, num_splits=3)
    S.sa_set_debug_validate(True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    # the other calls pass too on valid data
    mu = S.sa_page_summary(kv)
    S.sa_select_pages(kv, n_q_heads=wl.n_q_heads, mode=S.SA_SEL_PER_KV_HEAD, sink_pages=wl.sink_pages,
                      window_pages=wl.window_pages, top_k=wl.top_k, q=inp["q"], page_summary=mu)
    S.sa_select_decode(kv, inp["q"], mu, sink_pages=wl.sink_pages, window_pages=wl.window_pages, top_k=wl.top_k,
                       sm_scale=wl.sm_scale)
    torch.cuda.synchronize()


def test_list_entry_out_of_range(validating):
    wl, inp, lists, counts, _, npg = _decode_case()
    kv = _kv(inp, wl)
    bad = lists.copy()
    bad[1, 0, 2] = npg[1] + 5
    gl, gc = torch.from_numpy(bad).to(DEV), torch.from_numpy(counts).to(DEV)
    out = torch.full((wl.batch, 1, wl.n_q_heads, wl.d_v), 7.0, dtype=torch.bfloat16, device=DEV)
    _expect_data_error(lambda: S.sa_sparse_decode(kv, inp["q"], gl, gc, mode=S.SA_SEL_PER_KV_HEAD,
                                                  sm_scale=wl.sm_scale, num_splits=2, out=out),
                       "page_lists[1][0][2]")
    _expect_data_error(lambda: S.sa_sparse_decode_noalloc(kv, inp["q"], gl, gc, mode=S.SA_SEL_PER_KV_HEAD,
                                                          sm_scale=wl.sm_scale, num_splits=2, out=out),
                       "page_lists[1][0][2]")
    torch.cuda.synchronize()
    assert (out.float() == 7.0).all(), "an output was written"


def test_count_beyond_stride(validating):
    wl, inp, lists, counts, _, _ = _decode_case()
    kv = _kv(inp, wl)
    bad = counts.copy()
    bad[2, 1] = lists.shape[-1] + 1
    _expect_data_error(lambda: S.sa_sparse_decode(kv, inp["q"], torch.from_numpy(lists).to(DEV),
                                                  torch.from_numpy(bad).to(DEV), mode=S.SA_SEL_PER_KV_HEAD,
                                                  sm_scale=wl.sm_scale), "page_counts[2][1]")


def test_critical_count_beyond_count(validating):
    wl, inp, lists, counts, cc, _ = _decode_case("mla_tiered_decode_small", seed=62)
    kv = _kv(inp, wl)
    bad = cc.copy()
    bad[0, 0] = counts[0, 0] + 1
    _expect_data_error(lambda: S.sa_sparse_decode(kv, inp["q"], torch.from_numpy(lists).to(DEV),
                                                  torch.from_numpy(counts).to(DEV), mode=S.SA_SEL_PER_KV_HEAD,
                                                  sm_scale=wl.sm_scale, critical_counts=torch.from_numpy(bad).to(DEV),
                                                  ambient_head_mask=inp["ambient_mask"]), "critical_counts[0][0]")


def test_block_table_and_length_out_of_range(validating):
    wl, inp, lists, counts, _, _ = _decode_case()
    bt = inp["block_table"].clone()
    bt[0, 3] = inp["k_pool"].shape[0] + 100
    kv = _kv(inp, wl, block_table=bt)
    _expect_data_error(lambda: S.sa_page_summary(kv), "block_table[0][3]")
    mu = torch.zeros((inp["k_pool"].shape[0], wl.n_kv_heads, wl.d_qk), dtype=torch.float32, device=DEV)
    _expect_data_error(lambda: S.sa_select_pages(kv, n_q_heads=wl.n_q_heads, mode=S.SA_SEL_PER_KV_HEAD,
                                                 sink_pages=wl.sink_pages, window_pages=wl.window_pages,
                                                 top_k=wl.top_k, q=inp["q"], page_summary=mu), "block_table[0][3]")
    _expect_data_error(lambda: S.sa_select_decode(kv, inp["q"], mu, sink_pages=wl.sink_pages,
                                                  window_pages=wl.window_pages, top_k=wl.top_k,
                                                  sm_scale=wl.sm_scale), "block_table[0][3]")
    lens = inp["seq_lens"].clone()
    lens[2] = -4
    _expect_data_error(lambda: S.sa_page_summary(_kv(inp, wl, seq_lens=lens)), "seq_lens[2]")


def test_given_scores_not_finite(validating):
    wl, inp, _, _, _, _ = _decode_case("token_head_decode_small", seed=63)
    kv = _kv(inp, wl)
    sc = inp["scores"].clone()
    sc[1, 3, 17] = float("inf")
    _expect_data_error(lambda: S.sa_select_pages(kv, n_q_heads=wl.n_q_heads, mode=S.SA_SEL_PER_Q_HEAD,
                                                 sink_pages=0, window_pages=0, top_k=wl.top_k, scores=sc),
                       "scores[1][3][17]")


def test_prefill_block_table_out_of_range(validating):
    pw = W.SMALL["chunked_prefill_small"]
    cpu = W.make_prefill_inputs(pw, "cpu", seed=64)
    inp = {k: v.to(DEV) for k, v in cpu.items()}
    bt = inp["block_table"].clone()
    bt[0, 5] = -3
    kv = S.PagedKV(inp["k_pool"], inp["v_pool"], bt, inp["seq_lens"])
    _expect_data_error(lambda: S.sa_block_sparse_prefill(kv, 0, inp["q"], pw.q_start, inp["block_mask"], pw.block_q,
                                                         pw.sm_scale), "block_table[0][5]")
