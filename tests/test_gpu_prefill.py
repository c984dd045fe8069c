"""HIP block-sparse chunked prefill (GQA-union block tables, then causal
attention in place over the paged KV) against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle.sparse_attn_oracle as O
import sparse_attention_long_page_amd as S
import workloads as W
from _parity import compare_outputs, np64, npi

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def gpu_inputs(cpu):
    return {k: v.to(DEV) for k, v in cpu.items()}


def run_gpu(inp, wl):
    kv = S.PagedKV(inp["k_pool"], inp["v_pool"], inp["block_table"], inp["seq_lens"])
    out, lse, table, counts = S.sa_block_sparse_prefill(kv, 0, inp["q"], wl.q_start, inp["block_mask"],
                                                        wl.block_q, wl.sm_scale)
    torch.cuda.synchronize()
    return out, lse, table, counts


def check_tables(table, counts, mask, n_kv_heads):
    o_tab, o_cnt = O.gqa_union_block_table(npi(mask), n_kv_heads)
    t, c = npi(table), npi(counts)
    assert np.array_equal(c, o_cnt), (c, o_cnt)
    for g in range(n_kv_heads):
        assert np.array_equal(t[g, :c[g]], o_tab[g, :o_cnt[g]]), f"group {g} table differs"
    return o_tab, o_cnt


def oracle_prefill(cpu, wl, tab, cnt, rows=None):
    return O.block_sparse_prefill(np64(cpu["q"]), np64(cpu["k_pool"]), np64(cpu["v_pool"]),
                                  npi(cpu["block_table"])[0], int(npi(cpu["seq_lens"])[0]), wl.page_size,
                                  wl.q_start, tab, cnt, wl.n_kv_heads, wl.sm_scale, rows=rows)


SMALL = W.SMALL["chunked_prefill_small"]
CASES = {
    # ragged query tail (200 = 3*64 + 8), chunk start inside a page, extra pool pages
    "random_g4": SMALL,
    "ones_g4": SMALL.replace(mask_kind="ones"),
    "shared_g4": SMALL.replace(mask_kind="shared_columns", random_fraction=0.25),
    # group sizes 1, 2 and 8 take the other workgroup shapes (8: two workgroups per group)
    "random_g1": SMALL.replace(n_q_heads=2, n_kv_heads=2),
    "random_g2": SMALL.replace(n_q_heads=4, n_kv_heads=2, q_len=130, q_start=64 * 9),
    "random_g8": SMALL.replace(n_q_heads=8, n_kv_heads=1, q_len=64, q_start=64 * 12 + 63),
    # odd and non-power-of-two groups: 3 (one head per workgroup, three per
    # tile) and 6 (two heads per workgroup, three per tile)
    "random_g3": SMALL.replace(n_q_heads=6, n_kv_heads=2, q_len=150, q_start=64 * 7 + 5),
    "random_g6": SMALL.replace(n_q_heads=6, n_kv_heads=1, q_len=100, q_start=64 * 10),
    # chunk at the start of the sequence: no prefix at all
    "start_g4": SMALL.replace(q_len=150, q_start=0),
    # chunk shorter than one tile
    "short_g4": SMALL.replace(q_len=5, q_start=777),
}


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_matches_oracle(name):
    wl = CASES[name]
    cpu = W.make_prefill_inputs(wl, "cpu", seed=21)
    inp = gpu_inputs(cpu)
    out, lse, table, counts = run_gpu(inp, wl)
    tab, cnt = check_tables(table, counts, cpu["block_mask"], wl.n_kv_heads)
    ref_o, ref_l = oracle_prefill(cpu, wl, tab, cnt)
    mx, mean, le = compare_outputs(out, lse, ref_o, ref_l)
    print(f"{name}: max_abs {mx:.3e} mean_abs {mean:.3e} lse {le:.3e} counts {cnt.tolist()}")


def test_prefill_empty_group_and_unreachable_rows():
    """A group whose table is empty gives o = 0 and lse = -inf; a table with
    only blocks past some rows' positions leaves exactly those rows empty."""
    wl = SMALL.replace(q_len=100, q_start=640)
    cpu = W.make_prefill_inputs(wl, "cpu", seed=22)
    mask = torch.zeros_like(cpu["block_mask"])
    # group 1 keeps only the last KV block (position 704..): rows before it see nothing
    last = wl.n_kv_blocks - 1
    mask[wl.group:, :, last] = 1
    cpu["block_mask"] = mask
    inp = gpu_inputs(cpu)
    out, lse, table, counts = run_gpu(inp, wl)
    tab, cnt = check_tables(table, counts, mask, wl.n_kv_heads)
    assert cnt.tolist() == [0, 1]
    o = out.float().cpu()
    l = lse.cpu()
    assert (o[:, :wl.group] == 0).all() and torch.isneginf(l[:, :wl.group]).all()
    ref_o, ref_l = oracle_prefill(cpu, wl, tab, cnt)
    compare_outputs(out, lse, ref_o, ref_l)
    first_visible = last * wl.page_size - wl.q_start
    assert torch.isneginf(l[:first_visible, wl.group:]).all()
    assert torch.isfinite(l[first_visible:, wl.group:]).all()


def test_prefill_pool_permutation_invariant_and_deterministic():
    wl = SMALL
    cpu = W.make_prefill_inputs(wl, "cpu", seed=23)
    inp = gpu_inputs(cpu)
    a = run_gpu(inp, wl)
    b = run_gpu(inp, wl)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    n_phys = inp["k_pool"].shape[0]
    perm = torch.randperm(n_phys, generator=torch.Generator().manual_seed(3)).to(DEV)
    k2 = torch.empty_like(inp["k_pool"]); k2[perm] = inp["k_pool"]
    v2 = torch.empty_like(inp["v_pool"]); v2[perm] = inp["v_pool"]
    bt = inp["block_table"]
    inp2 = dict(inp, k_pool=k2, v_pool=v2,
                block_table=torch.where(bt >= 0, perm[bt.clamp(min=0).long()].to(torch.int32), bt).contiguous())
    c = run_gpu(inp2, wl)
    assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1])


def test_full_size_chunked_prefill_128k_sampled():
    """Full-size chunk (2048 queries at 126976 over 129024 KV tokens, 32/8 heads):
    block tables bit-exact; attention on every row of the first and last
    Q-block for all heads, plus 256 seeded random (query, head) rows."""
    wl = W.CHUNKED_PREFILL_128K
    inp = W.make_prefill_inputs(wl, DEV, seed=31)
    out, lse, table, counts = run_gpu(inp, wl)
    tab, cnt = check_tables(table, counts, inp["block_mask"].cpu(), wl.n_kv_heads)
    rng = np.random.default_rng(31)
    rows = set()
    # every row of the first and the last Q-block, for every head
    for h in range(wl.n_q_heads):
        for i in list(range(0, wl.block_q)) + list(range(wl.q_len - wl.block_q, wl.q_len)):
            rows.add((i, h))
    for i, h in zip(rng.integers(0, wl.q_len, 256), rng.integers(0, wl.n_q_heads, 256)):
        rows.add((int(i), int(h)))
    rows = sorted(rows)
    cpu = {k: v.cpu() for k, v in inp.items()}
    ref_o, ref_l = oracle_prefill(cpu, wl, tab, cnt, rows=rows)
    sel = np.zeros((wl.q_len, wl.n_q_heads), dtype=bool)
    for i, h in rows:
        sel[i, h] = True
    mx, mean, le = compare_outputs(out, lse, ref_o, ref_l, rows_mask=sel)
    print(f"full-size prefill: {len(rows)} rows max_abs {mx:.3e} mean_abs {mean:.3e} lse {le:.3e} "
          f"union blocks {cnt.tolist()} of {wl.n_kv_blocks}")
