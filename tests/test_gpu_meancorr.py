"""HIP mean correction of a block-sparse prefill (the skipped causal blocks
re-enter as mean terms) and the per-page mean value rows it needs, against
the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle.sparse_attn_oracle as O
import sparse_attention_long_page_amd as S
import workloads as W
from _parity import compare_outputs, np64, npi, oracle_pools

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def gpu_inputs(cpu):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in cpu.items()}


# ------------------------------------------------------------ value means
SUMMARY_CASES = ["bf16_d128_p16_kv_small", "bf16_d64_p64_q_small", "fp32_d64_p16_q_small",
                 "fp32_d128_p64_kv_small", "fp8_d128_p64_kv_small", "llama3_decode_small"]


@pytest.mark.parametrize("name", SUMMARY_CASES)
def test_value_summary_matches_oracle(name):
    wl = W.SMALL[name]
    inp = W.make_decode_inputs(wl, DEV, seed=41)
    kv = S.PagedKV(inp["k_pool"], inp["v_pool"], inp["block_table"], inp["seq_lens"],
                   k_scale=inp.get("k_scale"), v_scale=inp.get("v_scale"))
    nu = S.sa_page_value_summary(kv)
    torch.cuda.synchronize()
    _, vp = oracle_pools({k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()})
    ref = O.page_value_summary(vp, npi(inp["block_table"]), npi(inp["seq_lens"]), wl.page_size)
    got = nu.cpu().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "written pages differ"
    m = ~np.isnan(ref)
    # float64 sums in another order, both rounded once to fp32: at most one ulp apart
    err = np.abs(got[m].astype(np.float64) - ref[m].astype(np.float64))
    assert np.all(err <= np.spacing(np.abs(ref[m])).astype(np.float64) + 1e-30), float(err.max())


def test_value_summary_last_pages_only():
    wl = W.SMALL["bf16_d128_p16_kv_small"]
    inp = W.make_decode_inputs(wl, DEV, seed=42)
    kv = S.PagedKV(inp["k_pool"], inp["v_pool"], inp["block_table"], inp["seq_lens"])
    full = S.sa_page_value_summary(kv)
    last = S.sa_page_value_summary(kv, last_pages=1)
    torch.cuda.synchronize()
    bt, lens = npi(inp["block_table"]), npi(inp["seq_lens"])
    newest = {int(bt[b, (int(lens[b]) + wl.page_size - 1) // wl.page_size - 1])
              for b in range(lens.shape[0]) if lens[b] > 0}
    f, l = full.cpu(), last.cpu()
    for p in range(f.shape[0]):
        if p in newest:
            assert torch.equal(f[p], l[p])
        else:
            assert torch.isnan(l[p]).all()


# -------------------------------------------------------- mean correction
SMALL = W.SMALL["chunked_prefill_small"]
CASES = {
    "random_g4": SMALL,
    # few shared columns: most causal blocks are skipped and re-enter as means
    "shared_g4": SMALL.replace(mask_kind="shared_columns", random_fraction=0.15),
    "shared_g1": SMALL.replace(n_q_heads=2, n_kv_heads=2, mask_kind="shared_columns", random_fraction=0.1),
    "shared_g8": SMALL.replace(n_q_heads=8, n_kv_heads=1, q_len=64, q_start=64 * 12 + 63,
                               mask_kind="shared_columns", random_fraction=0.2),
    "shared_start": SMALL.replace(q_len=150, q_start=0, mask_kind="shared_columns", random_fraction=0.1),
    "shared_short": SMALL.replace(q_len=5, q_start=777, mask_kind="shared_columns", random_fraction=0.1),
    # 3 and 6 heads per KV head: query tiles of 80 and 32 over 8 and 6 waves
    "shared_g3": SMALL.replace(n_q_heads=6, n_kv_heads=2, mask_kind="shared_columns", random_fraction=0.1),
    "shared_g6": SMALL.replace(n_q_heads=6, n_kv_heads=1, q_len=90, mask_kind="shared_columns",
                               random_fraction=0.1),
    # more skipped blocks than one 32-block chunk
    "long_prefix": SMALL.replace(q_len=70, q_start=64 * 40 + 5, mask_kind="shared_columns",
                                 random_fraction=0.05),
}


def run_corrected(inp, wl):
    """Prefill, both page summaries, then the correction; returns the
    prefill's (o, lse) copy, the corrected (o, lse), tables and counts."""
    kv = S.PagedKV(inp["k_pool"], inp["v_pool"], inp["block_table"], inp["seq_lens"])
    out, lse, table, counts = S.sa_block_sparse_prefill(kv, 0, inp["q"], wl.q_start, inp["block_mask"],
                                                        wl.block_q, wl.sm_scale)
    base = (out.clone(), lse.clone())
    mu = S.sa_page_summary(kv)
    nu = S.sa_page_value_summary(kv)
    S.sa_prefill_mean_correction(kv, 0, inp["q"], wl.q_start, table, counts, mu, nu, wl.sm_scale, out, lse)
    torch.cuda.synchronize()
    return base, (out, lse), npi(table), npi(counts)


def oracle_corrected(cpu, wl, tab, cnt, rows=None):
    return O.mean_corrected_prefill(np64(cpu["q"]), np64(cpu["k_pool"]), np64(cpu["v_pool"]),
                                    npi(cpu["block_table"])[0], int(npi(cpu["seq_lens"])[0]), wl.page_size,
                                    wl.q_start, tab, cnt, wl.n_kv_heads, wl.sm_scale, rows=rows)


def n_skipped(wl, seq_len, tab, cnt):
    n_seq = (seq_len + wl.page_size - 1) // wl.page_size
    return [n_seq - len(set(tab[g, :cnt[g]].tolist())) for g in range(wl.n_kv_heads)]


@pytest.mark.parametrize("name", list(CASES))
def test_mean_correction_matches_oracle(name):
    wl = CASES[name]
    cpu = W.make_prefill_inputs(wl, "cpu", seed=51)
    inp = gpu_inputs(cpu)
    _, (out, lse), tab, cnt = run_corrected(inp, wl)
    ref_o, ref_l = oracle_corrected(cpu, wl, tab, cnt)
    mx, mean, le = compare_outputs(out, lse, ref_o, ref_l)
    print(f"{name}: max_abs {mx:.3e} mean_abs {mean:.3e} lse {le:.3e} "
          f"skipped {n_skipped(wl, int(npi(cpu['seq_lens'])[0]), tab, cnt)}")


def test_mean_correction_no_skip_is_identity():
    """Every causal block kept: nothing to add, (o, lse) stay bit for bit."""
    wl = SMALL.replace(mask_kind="ones")
    inp = gpu_inputs(W.make_prefill_inputs(wl, "cpu", seed=52))
    base, (out, lse), _, _ = run_corrected(inp, wl)
    assert torch.equal(base[0], out) and torch.equal(base[1], lse)


def test_mean_correction_exact_on_constant_blocks():
    """When every block's tokens share one key and one value, the mean term of
    a skipped block is that block exactly: the corrected result is dense
    causal attention (the oracle's block_sparse_prefill over all blocks)."""
    wl = CASES["shared_g4"]
    cpu = W.make_prefill_inputs(wl, "cpu", seed=53)
    cpu["k_pool"] = cpu["k_pool"][:, :, :1, :].expand_as(cpu["k_pool"]).contiguous()
    cpu["v_pool"] = cpu["v_pool"][:, :, :, :1].expand_as(cpu["v_pool"]).contiguous()
    inp = gpu_inputs(cpu)
    _, (out, lse), tab, cnt = run_corrected(inp, wl)
    nkb = wl.n_kv_blocks
    dense_tab = np.tile(np.arange(nkb, dtype=np.int32), (wl.n_kv_heads, 1))
    dense_cnt = np.full(wl.n_kv_heads, nkb, dtype=np.int32)
    ref_o, ref_l = O.block_sparse_prefill(np64(cpu["q"]), np64(cpu["k_pool"]), np64(cpu["v_pool"]),
                                          npi(cpu["block_table"])[0], int(npi(cpu["seq_lens"])[0]),
                                          wl.page_size, wl.q_start, dense_tab, dense_cnt, wl.n_kv_heads,
                                          wl.sm_scale)
    mx, mean, le = compare_outputs(out, lse, ref_o, ref_l)
    print(f"constant blocks vs dense: max_abs {mx:.3e} lse {le:.3e}")


def test_mean_correction_empty_table_rows():
    """A group with an empty table: rows that reach no whole block stay empty
    (o = 0, lse = -inf); the rest are the mean terms alone."""
    wl = SMALL.replace(q_len=100, q_start=640)
    cpu = W.make_prefill_inputs(wl, "cpu", seed=54)
    cpu["block_mask"] = torch.zeros_like(cpu["block_mask"])
    inp = gpu_inputs(cpu)
    _, (out, lse), tab, cnt = run_corrected(inp, wl)
    assert cnt.tolist() == [0] * wl.n_kv_heads
    ref_o, ref_l = oracle_corrected(cpu, wl, tab, cnt)
    compare_outputs(out, lse, ref_o, ref_l)
    assert torch.isfinite(lse).all()          # block 0 lies wholly before position 640


def test_full_size_chunked_prefill_128k_mean_correction_sampled():
    """Full-size chunk (2048 queries at 126976, 32/8 heads) with shared
    columns (most of the 2000+ causal blocks skipped): 96 seeded rows against
    the oracle, including the first and last query of the chunk."""
    wl = W.CHUNKED_PREFILL_128K.replace(mask_kind="shared_columns", random_fraction=0.1)
    inp = W.make_prefill_inputs(wl, DEV, seed=55)
    _, (out, lse), tab, cnt = run_corrected(inp, wl)
    rng = np.random.default_rng(55)
    rows = {(0, 0), (wl.q_len - 1, wl.n_q_heads - 1)}
    for i, h in zip(rng.integers(0, wl.q_len, 94), rng.integers(0, wl.n_q_heads, 94)):
        rows.add((int(i), int(h)))
    rows = sorted(rows)
    cpu = {k: v.cpu() for k, v in inp.items()}
    ref_o, ref_l = oracle_corrected(cpu, wl, tab, cnt, rows=rows)
    sel = np.zeros((wl.q_len, wl.n_q_heads), dtype=bool)
    for i, h in rows:
        sel[i, h] = True
    mx, mean, le = compare_outputs(out, lse, ref_o, ref_l, rows_mask=sel)
    print(f"full-size mean correction: {len(rows)} rows max_abs {mx:.3e} lse {le:.3e} "
          f"skipped {n_skipped(wl, int(npi(cpu['seq_lens'])[0]), tab, cnt)}")


def test_mean_correction_rejects_bad_arguments():
    wl = SMALL
    inp = gpu_inputs(W.make_prefill_inputs(wl, "cpu", seed=56))
    kv = S.PagedKV(inp["k_pool"], inp["v_pool"], inp["block_table"], inp["seq_lens"])
    out, lse, table, counts = S.sa_block_sparse_prefill(kv, 0, inp["q"], wl.q_start, inp["block_mask"],
                                                        wl.block_q, wl.sm_scale)
    mu = S.sa_page_summary(kv)
    nu = S.sa_page_value_summary(kv)
    with pytest.raises(S.SparseAttnError):
        S.sa_prefill_mean_correction(kv, 0, inp["q"], wl.q_start, table, counts, mu, nu, -1.0, out, lse)
    with pytest.raises(S.SparseAttnError):      # workspace one byte short
        need = S.sa_prefill_mean_correction_workspace_size(kv, table.shape[-1])
        S.sa_prefill_mean_correction(kv, 0, inp["q"], wl.q_start, table, counts, mu, nu, wl.sm_scale, out, lse,
                                     workspace=torch.empty(need - 1, dtype=torch.uint8, device=DEV))
    with pytest.raises(S.SparseAttnError):      # table too short to cover the chunk
        S.sa_prefill_mean_correction(kv, 0, inp["q"], wl.q_start, table[:, :3].contiguous(), counts, mu, nu,
                                     wl.sm_scale, out, lse)
    torch.cuda.synchronize()
