"""sa_sparse_decode_noalloc (split partials in the library's static device
scratch) against sa_sparse_decode (caller workspace), through the C ABI: the
same outputs bit for bit, and within the oracle's tolerance, on two calls in a
row whose second has the smaller input (the scratch keeps the first call's
partials, which the second must not read)."""
import numpy as np
import pytest
import torch

import oracle.sparse_attn_oracle as O
import sparse_attention_long_page_amd as S
import workloads as W
from _parity import compare_outputs, np64, npi

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(wl, seed):
    cpu = W.make_decode_inputs(wl, "cpu", seed=seed)
    inp = {k: (v.to(DEV) if v is not None else None) for k, v in cpu.items()}
    kv = S.PagedKV(inp["k_pool"], inp["v_pool"], inp["block_table"], inp["seq_lens"], d_v=wl.d_v)
    bt, lens = npi(cpu["block_table"]), npi(cpu["seq_lens"])
    npg = [O.n_pages_of(L, wl.page_size) for L in lens]
    mu = O.page_summary(np64(cpu["k_pool"]), bt, lens, wl.page_size)
    sc = O.page_scores(np64(cpu["q"]), mu, bt, lens, wl.page_size, wl.n_kv_heads, wl.mode)
    lists, counts, cc = O.select_pages(sc, npg, wl.sink_pages, wl.window_pages, wl.top_k, wl.critical_k)
    return cpu, inp, kv, lists, counts, cc


def _both(wl, seed, splits):
    cpu, inp, kv, lists, counts, cc = _case(wl, seed)
    args = dict(mode=S.SA_SEL_PER_KV_HEAD if wl.mode == "per_kv_head" else S.SA_SEL_PER_Q_HEAD,
                sm_scale=wl.sm_scale, num_splits=splits,
                critical_counts=None if cc is None else torch.from_numpy(cc).to(DEV),
                ambient_head_mask=inp["ambient_mask"])
    gl, gc = torch.from_numpy(lists).to(DEV), torch.from_numpy(counts).to(DEV)
    ref = S.sa_sparse_decode(kv, inp["q"], gl, gc, **args)
    got = S.sa_sparse_decode_noalloc(kv, inp["q"], gl, gc, **args)
    torch.cuda.synchronize()
    assert torch.equal(got[0], ref[0]), "output differs from sa_sparse_decode"
    assert torch.equal(got[1], ref[1]), "lse differs from sa_sparse_decode"
    amask = None if inp["ambient_mask"] is None else npi(cpu["ambient_mask"]).astype(np.int64) & 0xffffffff
    ref_o, ref_l = O.sparse_decode(np64(cpu["q"]), np64(cpu["k_pool"]),
                                   None if cpu["v_pool"] is None else np64(cpu["v_pool"]),
                                   npi(cpu["block_table"]), npi(cpu["seq_lens"]), wl.page_size, lists, counts,
                                   wl.n_kv_heads, wl.mode, wl.sm_scale, cc, amask, d_v=wl.d_v)
    compare_outputs(got[0], got[1], ref_o, ref_l, fp32=wl.dtype == "fp32")


@pytest.mark.parametrize("name", ["llama3_decode_small", "token_head_decode_small", "mla_tiered_decode_small"])
def test_noalloc_equals_workspace_decode_on_two_calls(name):
    big = W.SMALL[name]
    if big.scores == "gumbel":
        big = big.replace(scores="summary", sink_pages=1, window_pages=2)
    small = big.replace(batch=1, seq_lens=None if big.seq_lens is None else big.seq_lens[1:2])
    _both(big, seed=41, splits=3)       # first call: larger input
    _both(small, seed=42, splits=2)     # second call: smaller input, fewer splits


def test_noalloc_without_partials():
    """One split needs no scratch: the call never looks the array up."""
    _both(W.SMALL["llama3_decode_small"], seed=43, splits=1)
