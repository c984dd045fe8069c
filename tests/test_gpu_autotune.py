"""HIP AutoTuner of the tiered selection against the CPU oracle, through the C
ABI: the estimated (query head, page) attention mass, the coverage of every
(alpha, h) configuration with the configuration kept, and the Ambient head
mask."""
import numpy as np
import pytest
import torch

import oracle.sparse_attn_oracle as O
import sparse_attention_long_page_amd as S
import workloads as W
from _parity import np64, npi, oracle_pools, sub_pool

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def kv_of(inp):
    return S.PagedKV(inp["k_pool"], inp["v_pool"], inp["block_table"], inp["seq_lens"],
                     k_scale=inp.get("k_scale"), v_scale=inp.get("v_scale"))


def cpu_of(inp):
    return {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


# ------------------------------------------------------------- head mass
def check_mass(got, ref, lens, P, T):
    """Masses within 1e-3 relative + 1e-6 absolute of the oracle (fp32
    softmax over fp32-accurate logits); each head's masses sum to T."""
    worst = 0.0
    for b, L in enumerate(lens):
        n = (int(L) + P - 1) // P
        g, r = got[b, :, :n].astype(np.float64), ref[b, :, :n]
        err = np.abs(g - r)
        assert np.all(err <= 1e-3 * r + 1e-6), float((err - 1e-3 * r).max())
        assert np.allclose(g.sum(axis=1), T, atol=1e-4)
        worst = max(worst, float(err.max()) if err.size else 0.0)
    return worst


MASS_CASES = ["mla_tiered_decode_small", "llama3_decode_small", "bf16_d64_p16_kv_small",
              "bf16_d128_p64_q_small", "fp8_d128_p64_kv_small", "token_head_decode_small"]


@pytest.mark.parametrize("name", MASS_CASES)
def test_head_mass_matches_oracle(name):
    wl = W.SMALL[name]
    inp = W.make_decode_inputs(wl, DEV, seed=61)
    kv = kv_of(inp)
    mu = S.sa_page_summary(kv)
    M = S.sa_head_page_mass(kv, inp["q"], mu, wl.sm_scale)
    torch.cuda.synchronize()
    cpu = cpu_of(inp)
    kp, _ = oracle_pools(cpu)
    lens = npi(cpu["seq_lens"])
    bt = npi(cpu["block_table"])
    mu_o = O.page_summary(kp, bt, lens, wl.page_size)
    ref = O.head_page_mass(np64(cpu["q"]), mu_o, bt, lens, wl.page_size, wl.n_kv_heads, wl.sm_scale)
    worst = check_mass(M.cpu().numpy(), ref, lens, wl.page_size, wl.q_tokens)
    print(f"{name}: max abs mass err {worst:.2e}")


def test_full_size_mla_head_mass_sampled():
    """Full-size MLA decode (16 sequences of 65536 tokens, 128 heads, 2 query
    tokens, latent d 576): the first and last sequences' masses against the
    oracle on their own pages."""
    wl = W.MLA_TIERED_DECODE_64K
    inp = W.make_decode_inputs(wl, DEV, seed=62)
    kv = kv_of(inp)
    mu = S.sa_page_summary(kv)
    M = S.sa_head_page_mass(kv, inp["q"], mu, wl.sm_scale)
    torch.cuda.synchronize()
    pick = [0, wl.batch - 1]
    kp, _, nbt, lens = sub_pool(inp, pick)
    mu_o = O.page_summary(kp, nbt, lens, wl.page_size)
    q = np64(inp["q"][pick].cpu())
    ref = O.head_page_mass(q, mu_o, nbt, lens, wl.page_size, wl.n_kv_heads, wl.sm_scale)
    worst = check_mass(M[pick].cpu().numpy(), ref, lens, wl.page_size, wl.q_tokens)
    print(f"full-size MLA head mass: max abs err {worst:.2e}")


# ------------------------------------------------------------- coverage
def synthetic_tier_inputs(seed, B, Hkv, G, T, P, lens, max_pages, ties=True):
    """Seeded masses (positive, each head's masses sum to T) and router
    scores (small integers, so ranks tie and the index breaks them)."""
    rng = np.random.default_rng(seed)
    Hq = Hkv * G
    M = np.full((B, Hq, max_pages), np.nan, dtype=np.float32)
    scores = np.full((B, Hkv, max_pages), np.nan, dtype=np.float32)
    for b, L in enumerate(lens):
        n = (L + P - 1) // P
        if n == 0:
            continue
        raw = rng.random((Hq, n)) ** 4
        M[b, :, :n] = (T * raw / raw.sum(axis=1, keepdims=True)).astype(np.float32)
        sc = rng.integers(-4, 5, size=(Hkv, n)) if ties else rng.standard_normal((Hkv, n))
        scores[b, :, :n] = sc.astype(np.float32)
    return M, scores


def fake_kv(B, Hkv, P, lens, max_pages):
    """A cache descriptor whose pools are never read (the tuner reads only the
    sequence lengths and sizes)."""
    n_phys = max(1, sum((L + P - 1) // P for L in lens))
    k = torch.zeros((n_phys, Hkv, P, 64), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros((n_phys, Hkv, 64, P), dtype=torch.bfloat16, device=DEV)
    bt = torch.full((B, max_pages), -1, dtype=torch.int32)
    off = 0
    for b, L in enumerate(lens):
        n = (L + P - 1) // P
        bt[b, :n] = torch.arange(off, off + n, dtype=torch.int32)
        off += n
    return S.PagedKV(k, v, bt.to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV))


def check_tuner(M, scores, lens, P, Hkv, T, sink, window, budget, alphas, heads):
    B, Hq, max_pages = M.shape
    kv = fake_kv(B, Hkv, P, lens, max_pages)
    cov, choice = S.sa_autotune_tiers(kv, torch.from_numpy(M).to(DEV), torch.from_numpy(scores).to(DEV),
                                      q_tokens=T, sink_pages=sink, window_pages=window, budget=budget,
                                      alphas=alphas, ambient_heads=heads)
    torch.cuda.synchronize()
    rc, rbeta, rbest = O.tier_coverage(M.astype(np.float64), scores, np.array(lens), P, Hkv, T, sink, window,
                                       budget, alphas, heads)
    c = cov.cpu().numpy().astype(np.float64)
    ch = choice.cpu().numpy().tolist()
    assert np.array_equal(np.isnan(c), np.isnan(rc))
    ok = ~np.isnan(rc)
    assert np.all(np.abs(c[ok] - rc[ok]) <= 2e-6 + 2e-6 * np.abs(rc[ok])), float(np.abs(c[ok] - rc[ok]).max())
    if rbest is None:
        assert ch == [-1, -1, -1]
    else:
        # the kept configuration is a maximum up to the fp32 sums' rounding
        ia, ih = ch[0], ch[1]
        assert rc[ia, ih] >= rc[rbest] - 4e-6, (ch, rbest)
        assert ch[2] == rbeta[ia, ih]
        top = rc[rbest]
        if all(rc[i, j] < top - 4e-6 for i in range(len(alphas)) for j in range(len(heads))
               if ok[i, j] and (i, j) != rbest):
            assert (ia, ih) == rbest
    return c, ch


TUNER_CASES = {
    # GQA groups of 8, two KV heads, sink + window, a sequence shorter than the forced pages
    "g8_forced": dict(B=4, Hkv=2, G=8, T=2, P=16, lens=[16 * 37 + 5, 16 * 9, 40, 16 * 60], max_pages=64,
                      sink=1, window=2, budget=64, alphas=[0, 2, 4, 8, 64], heads=[1, 2, 4, 8]),
    # MLA shape: 128 heads per KV head, no forced pages, infeasible alphas in the grid
    "g128_mla": dict(B=3, Hkv=1, G=128, T=2, P=64, lens=[64 * 300 + 7, 64 * 128, 64 * 50], max_pages=320,
                     sink=0, window=0, budget=2048, alphas=[0, 4, 8, 12, 16, 17], heads=[16, 32, 64, 128]),
    # nothing feasible
    "none_feasible": dict(B=2, Hkv=2, G=4, T=1, P=16, lens=[300, 200], max_pages=32, sink=0, window=1,
                          budget=3, alphas=[1, 2], heads=[1]),
}


@pytest.mark.parametrize("name", list(TUNER_CASES))
def test_autotune_matches_oracle(name):
    c = TUNER_CASES[name]
    M, scores = synthetic_tier_inputs(71, c["B"], c["Hkv"], c["G"], c["T"], c["P"], c["lens"], c["max_pages"])
    cov, ch = check_tuner(M, scores, c["lens"], c["P"], c["Hkv"], c["T"], c["sink"], c["window"], c["budget"],
                          c["alphas"], c["heads"])
    print(f"{name}: choice {ch} coverage max {np.nanmax(cov) if not np.all(np.isnan(cov)) else None}")


def test_full_size_autotune_mla_shape():
    """16 sequences of 1024 pages, 128 heads per KV head, 2 query tokens:
    the MLA decode's shape, with the default tier grid around its
    configuration (8 Critical pages, 32 Ambient heads)."""
    lens = [65536] * 16
    M, scores = synthetic_tier_inputs(72, 16, 1, 128, 2, 64, lens, 1024, ties=False)
    budget = 8 * 128 + 32 * 32
    cov, ch = check_tuner(M, scores, lens, 64, 1, 2, 0, 0, budget, [0, 4, 8, 12, 16], [16, 32, 64, 128])
    print(f"full-size tuner: choice {ch} coverage {cov.round(4).tolist()}")


# ------------------------------------------------------------ ambient mask
@pytest.mark.parametrize("G,h", [(8, 3), (4, 4), (128, 32), (32, 0)])
def test_ambient_mask_matches_oracle(G, h):
    """Integer masses (ties broken by head index), seeded tiered lists:
    the mask bit for bit."""
    rng = np.random.default_rng(81 + G + h)
    B, Hkv, P = 3, 2 if G < 128 else 1, 16
    Hq = G * Hkv
    lens = [16 * 40, 16 * 25 + 3, 16 * 9]
    max_pages, stride = 48, 20
    M = rng.integers(0, 6, size=(B, Hq, max_pages)).astype(np.float32)
    lists = np.full((B, Hkv, stride), -1, dtype=np.int32)
    counts = np.zeros((B, Hkv), dtype=np.int32)
    cc = np.zeros((B, Hkv), dtype=np.int32)
    for b, L in enumerate(lens):
        n = (L + P - 1) // P
        for g in range(Hkv):
            c = int(rng.integers(0, min(n, stride) + 1))
            crit = int(rng.integers(0, c + 1))
            pages = rng.permutation(n)[:c]
            lists[b, g, :crit] = np.sort(pages[:crit])
            lists[b, g, crit:c] = np.sort(pages[crit:])
            counts[b, g], cc[b, g] = c, crit
    kv = fake_kv(B, Hkv, P, lens, max_pages)
    mask = S.sa_ambient_head_mask(kv, torch.from_numpy(M).to(DEV), torch.from_numpy(lists).to(DEV),
                                  torch.from_numpy(counts).to(DEV), torch.from_numpy(cc).to(DEV), h)
    torch.cuda.synchronize()
    ref = O.ambient_head_mask(M.astype(np.float64), lists, counts, cc, Hkv, h)
    got = mask.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, ref)


# -------------------------------------------------------------- end to end
def test_autotune_end_to_end_mla_small():
    """The MLA decode's small case: mass on the GPU against the oracle's from
    the same queries and pool, the search over it with seeded router scores,
    then the kept configuration drives the tiered lists and the Ambient mask
    (h bits on every Ambient page), and the tiered decode runs on them."""
    wl = W.SMALL["mla_tiered_decode_small"]
    inp = W.make_decode_inputs(wl, DEV, seed=63)
    kv = kv_of(inp)
    mu = S.sa_page_summary(kv)
    M = S.sa_head_page_mass(kv, inp["q"], mu, wl.sm_scale)
    cpu = cpu_of(inp)
    kp, _ = oracle_pools(cpu)
    lens, bt = npi(cpu["seq_lens"]), npi(cpu["block_table"])
    mu_o = O.page_summary(kp, bt, lens, wl.page_size)
    ref_M = O.head_page_mass(np64(cpu["q"]), mu_o, bt, lens, wl.page_size, wl.n_kv_heads, wl.sm_scale)
    _, scores = synthetic_tier_inputs(64, wl.batch, 1, wl.n_q_heads, wl.q_tokens, wl.page_size, lens.tolist(),
                                      wl.max_pages, ties=False)
    G = wl.n_q_heads
    budget = wl.critical_k * G + (wl.top_k - wl.critical_k) * wl.ambient_heads
    alphas, heads = [0, 1, 2, 3, 5], [4, 8, 16, 32]
    cov, choice = S.sa_autotune_tiers(kv, M, torch.from_numpy(scores).to(DEV), q_tokens=wl.q_tokens,
                                      sink_pages=0, window_pages=0, budget=budget, alphas=alphas,
                                      ambient_heads=heads)
    torch.cuda.synchronize()
    rc, rbeta, rbest = O.tier_coverage(ref_M, scores, lens, wl.page_size, 1, wl.q_tokens, 0, 0, budget, alphas,
                                       heads)
    c = cov.cpu().numpy().astype(np.float64)
    assert np.allclose(c, rc, atol=1e-4, equal_nan=True)
    ia, ih, beta = choice.cpu().tolist()
    assert rc[ia, ih] >= rc[rbest] - 1e-4 and beta == rbeta[ia, ih]
    # the kept configuration drives the tiered selection and its head mask
    alpha, h = alphas[ia], heads[ih]
    lists, counts, cc = S.sa_select_pages(kv, n_q_heads=G, mode=S.SA_SEL_PER_KV_HEAD, sink_pages=0, window_pages=0,
                                          top_k=alpha + beta, critical_k=alpha,
                                          scores=torch.from_numpy(scores).to(DEV))
    mask = S.sa_ambient_head_mask(kv, M, lists, counts, cc, h)
    torch.cuda.synchronize()
    m = mask.cpu().numpy().view(np.uint32)
    L, C, CC = lists.cpu().numpy(), counts.cpu().numpy(), cc.cpu().numpy()
    for b in range(wl.batch):
        amb = set(L[b, 0, CC[b, 0]:C[b, 0]].tolist())
        for p in range(wl.max_pages):
            bits = sum(bin(int(w)).count("1") for w in m[b, p])
            assert bits == (min(h, G) if p in amb else 0), (b, p, bits)
    out, lse = S.sa_sparse_decode(kv, inp["q"], lists, counts, mode=S.SA_SEL_PER_KV_HEAD, sm_scale=wl.sm_scale,
                                  critical_counts=cc, ambient_head_mask=mask)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    print(f"end to end: choice alpha {alpha} h {h} beta {beta} coverage {c[ia, ih]:.4f}")


def test_autotune_rejects_bad_arguments():
    lens = [100, 50]
    kv = fake_kv(2, 2, 16, lens, 8)
    M, scores = synthetic_tier_inputs(73, 2, 2, 4, 1, 16, lens, 8)
    Mt, st = torch.from_numpy(M).to(DEV), torch.from_numpy(scores).to(DEV)
    with pytest.raises(S.SparseAttnError):     # empty grid
        S.sa_autotune_tiers(kv, Mt, st, q_tokens=1, sink_pages=0, window_pages=0, budget=8, alphas=[],
                            ambient_heads=[1])
    with pytest.raises(S.SparseAttnError):     # h < 1
        S.sa_autotune_tiers(kv, Mt, st, q_tokens=1, sink_pages=0, window_pages=0, budget=8, alphas=[0],
                            ambient_heads=[0])
    with pytest.raises(S.SparseAttnError):     # scores stride below max_pages
        S.sa_autotune_tiers(kv, Mt, st[..., :4].contiguous(), q_tokens=1, sink_pages=0, window_pages=0, budget=8,
                            alphas=[0], ambient_heads=[1])
    torch.cuda.synchronize()
