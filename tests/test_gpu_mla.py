"""HIP tiered decode over a latent (MLA) cache -- Critical pages for every
query head, Ambient pages only for the heads in their head set -- against the
CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle.sparse_attn_oracle as O
import sparse_attention_long_page_amd as S
import workloads as W
from _parity import check_page_lists, compare_outputs, np64, npi
from test_gpu_decode import _full_size_check, gpu_inputs, gpu_select, make_kv, oracle_chain

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SMALL = W.SMALL["mla_tiered_decode_small"]


def _amask64(t):
    return npi(t).astype(np.int64) & 0xffffffff


def _oracle_decode(cpu, wl, lists, counts, cc, sm_scale=None):
    return O.sparse_decode(np64(cpu["q"]), np64(cpu["k_pool"]), None, npi(cpu["block_table"]),
                           npi(cpu["seq_lens"]), wl.page_size, lists, counts, wl.n_kv_heads, wl.mode,
                           wl.sm_scale if sm_scale is None else sm_scale, cc, _amask64(cpu["ambient_mask"]),
                           d_v=wl.d_v)


def test_mla_select_matches_oracle():
    """Head- and token-summed scores over 576-d page means, tiered top-k lists."""
    wl = SMALL
    cpu = W.make_decode_inputs(wl, "cpu", seed=31)
    inp = gpu_inputs(cpu)
    kv = make_kv(inp, wl)
    mu = S.sa_page_summary(kv)
    (lists, counts, cc), scores_out = gpu_select(inp, wl, kv, mu)
    torch.cuda.synchronize()
    _, o_scores, _, _, _, npg = oracle_chain(cpu, wl)
    g = scores_out.cpu().numpy()
    fin = ~np.isnan(o_scores)
    assert np.array_equal(np.isnan(g), ~fin)
    rel = np.abs(g[fin].astype(np.float64) - o_scores[fin]) / np.maximum(1.0, np.abs(o_scores[fin]))
    assert rel.max() <= 1e-6, rel.max()
    rep = check_page_lists(npi(lists), npi(counts), npi(cc), o_scores, npg, wl.sink_pages, wl.window_pages,
                           wl.top_k, wl.critical_k)
    assert not rep.failures, rep.failures[:5]


CASES = {
    # ragged last page (5 tokens), 32 heads: half of each 128-row workgroup is past the last head
    "small": SMALL,
    # one query token, 64 heads
    "t1": SMALL.replace(q_tokens=1, n_q_heads=64, ambient_heads=16),
    # four query tokens share each head's tile and Ambient bit
    "t4": SMALL.replace(q_tokens=4, n_q_heads=32, ambient_heads=5),
    # eight and sixteen query tokens per head (one head's rows fill half or all of a 16-row tile)
    "t8": SMALL.replace(q_tokens=8, n_q_heads=32, ambient_heads=9),
    "t16": SMALL.replace(q_tokens=16, n_q_heads=8, ambient_heads=3),
    # 144 heads: a second workgroup row group with only part of its rows valid
    "h144": SMALL.replace(n_q_heads=144, ambient_heads=40, batch=1),
    # no Ambient head at all for some pages' heads; no tiers beyond Critical
    "critical_only": SMALL.replace(top_k=4, critical_k=4, ambient_heads=3),
    # 256 heads, the most an Ambient head mask row holds (8 words): four row groups
    "h256": SMALL.replace(n_q_heads=256, ambient_heads=64, batch=1),
    # a split longer than the kernel's 128-page metadata window
    "long_split": SMALL.replace(batch=1, context=64 * 400 + 17, top_k=270, critical_k=30, ambient_heads=8),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("splits", [1, 3, 0])
def test_mla_decode_matches_oracle(name, splits):
    wl = CASES[name]
    cpu = W.make_decode_inputs(wl, "cpu", seed=32)
    inp = gpu_inputs(cpu)
    kv = make_kv(inp, wl)
    _, _, o_lists, o_counts, o_cc, _ = oracle_chain(cpu, wl)
    out, lse = S.sa_sparse_decode(kv, inp["q"], torch.from_numpy(o_lists).to(DEV),
                                  torch.from_numpy(o_counts).to(DEV), mode=S.SA_SEL_PER_KV_HEAD,
                                  sm_scale=wl.sm_scale, critical_counts=torch.from_numpy(o_cc).to(DEV),
                                  ambient_head_mask=inp["ambient_mask"], num_splits=splits)
    torch.cuda.synchronize()
    ref_o, ref_l = _oracle_decode(cpu, wl, o_lists, o_counts, o_cc)
    mx, mean, le = compare_outputs(out, lse, ref_o, ref_l)
    print(f"{name} splits {splits}: max_abs {mx:.3e} mean_abs {mean:.3e} lse {le:.3e}")


@pytest.mark.parametrize("splits", [1, 2])
@pytest.mark.parametrize("sm_scale", [1.0, 4.0])
def test_mla_large_logits_take_exact_max_pass(sm_scale, splits):
    """Logit ranges far beyond the first page's maximum (large softmax scale)
    exercise the exact-maximum fallback; the result must still match."""
    wl = SMALL
    cpu = W.make_decode_inputs(wl, "cpu", seed=33)
    inp = gpu_inputs(cpu)
    kv = make_kv(inp, wl)
    _, _, o_lists, o_counts, o_cc, _ = oracle_chain(cpu, wl)
    out, lse = S.sa_sparse_decode(kv, inp["q"], torch.from_numpy(o_lists).to(DEV),
                                  torch.from_numpy(o_counts).to(DEV), mode=S.SA_SEL_PER_KV_HEAD,
                                  sm_scale=sm_scale, critical_counts=torch.from_numpy(o_cc).to(DEV),
                                  ambient_head_mask=inp["ambient_mask"], num_splits=splits)
    torch.cuda.synchronize()
    ref_o, ref_l = _oracle_decode(cpu, wl, o_lists, o_counts, o_cc, sm_scale=sm_scale)
    # The softmax is nearly one-hot here, so outputs approach single V values
    # (|o| up to ~4, where one bf16 step is 2^-6 > 1e-2).  Each of three bf16
    # roundings moves an output by at most 2^-9 of the largest |v| the row
    # attends: of P before PV, of each split partial o_s (a convex combination
    # of V rows) before the merge, and of the output; the bar adds them to
    # 1e-2, with |v| bounded by the sequence's largest latent value.
    # Logits reach ~1e2-1e3, so lse is compared with a relative term too.
    g = np64(out)
    err = np.abs(g - ref_o)
    bt, lens = npi(cpu["block_table"]), npi(cpu["seq_lens"])
    kp = npi(cpu["k_pool"].float())
    for b in range(wl.batch):
        pages = bt[b, :O.n_pages_of(int(lens[b]), wl.page_size)]
        vmax = float(np.abs(kp[pages, 0, :, :wl.d_v]).max())
        assert (err[b] <= 1e-2 + 3 * 2.0 ** -9 * vmax).all(), (b, err[b].max(), vmax)
    assert err.mean() <= 1e-3, err.mean()
    gl = np64(lse)
    assert np.array_equal(np.isneginf(gl), np.isneginf(ref_l))
    fin = np.isfinite(ref_l)
    assert (np.abs(gl[fin] - ref_l[fin]) <= 2e-2 + 2e-5 * np.abs(ref_l[fin])).all()


def test_mla_empty_and_deterministic():
    wl = SMALL
    cpu = W.make_decode_inputs(wl, "cpu", seed=34)
    inp = gpu_inputs(cpu)
    kv = make_kv(inp, wl)
    _, _, o_lists, o_counts, o_cc, _ = oracle_chain(cpu, wl)
    lists, counts = torch.from_numpy(o_lists).to(DEV), torch.from_numpy(o_counts).to(DEV)
    cc = torch.from_numpy(o_cc).to(DEV)
    args = dict(mode=S.SA_SEL_PER_KV_HEAD, sm_scale=wl.sm_scale, critical_counts=cc,
                ambient_head_mask=inp["ambient_mask"], num_splits=3)
    a = S.sa_sparse_decode(kv, inp["q"], lists, counts, **args)
    b = S.sa_sparse_decode(kv, inp["q"], lists, counts, **args)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    # empty lists: o = 0, lse = -inf
    z = torch.zeros_like(counts)
    out, lse = S.sa_sparse_decode(kv, inp["q"], lists, z, **dict(args, critical_counts=z))
    torch.cuda.synchronize()
    assert (out.float() == 0).all() and torch.isneginf(lse).all()
    # Ambient pages with no head in the mask leave only the Critical pages
    none = torch.zeros_like(inp["ambient_mask"])
    out2, lse2 = S.sa_sparse_decode(kv, inp["q"], lists, counts, **dict(args, ambient_head_mask=none))
    torch.cuda.synchronize()
    ref_o, ref_l = O.sparse_decode(np64(cpu["q"]), np64(cpu["k_pool"]), None, npi(cpu["block_table"]),
                                   npi(cpu["seq_lens"]), wl.page_size, o_lists, o_cc, wl.n_kv_heads, wl.mode,
                                   wl.sm_scale, d_v=wl.d_v)
    compare_outputs(out2, lse2, ref_o, ref_l)


def test_full_size_mla_tiered_decode_64k_sampled():
    (mx, mean, lse_err), rep = _full_size_check(W.MLA_TIERED_DECODE_64K, seed=13, n_sample=2)
    print(f"max_abs {mx:.3e} mean_abs {mean:.3e} lse {lse_err:.3e} band events {rep.band_events}/{rep.units}")
