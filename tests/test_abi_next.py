"""Host-side argument checks of the mask producer, the mean correction and the
AutoTuner entry points: each bad argument is rejected with its status before
anything is launched (no GPU needed; no pointer is dereferenced)."""
import ctypes

import pytest

import sparse_attention_long_page_amd as S
from sparse_attention_long_page_amd import binding as B
from test_abi import FAKE, INV, UNS, WS, kv


def mask(kvd, **over):
    a = dict(seq=0, q=FAKE, q_len=128, q_start=64, n_q_heads=8, mu=FAKE, block_q=64, nkb=3, scale=0.1, top_k=2,
             max_gap=0.0, out=FAKE)
    a.update(over)
    return S.load_library().sa_prefill_block_mask(ctypes.byref(kvd), a["seq"], a["q"], a["q_len"], a["q_start"],
                                                   a["n_q_heads"], a["mu"], a["block_q"], a["nkb"], a["scale"],
                                                   a["top_k"], a["max_gap"], a["out"], None)


MASK_CASES = [
    ("latent cache", dict(kv=dict(v_pool=None, d_qk=576, d_v=512, n_kv_heads=1)), dict(n_q_heads=8), UNS),
    ("negative seq", {}, dict(seq=-1), INV),
    ("null summary", {}, dict(mu=None), INV),
    ("null out", {}, dict(out=None), INV),
    ("zero q_len", {}, dict(q_len=0), INV),
    ("zero block_q", {}, dict(block_q=0), INV),
    ("heads not multiple", {}, dict(n_q_heads=7), INV),
    ("group above 8", dict(kv=dict(n_kv_heads=1)), dict(n_q_heads=16), UNS),
    ("blocks short of the chunk", {}, dict(nkb=2), INV),
    ("blocks past max_pages", {}, dict(nkb=33), INV),
    ("scores over the LDS budget", dict(kv=dict(max_pages=8192)), dict(nkb=8192), UNS),
    ("zero scale", {}, dict(scale=0.0), INV),
    ("threshold mode, negative gap", {}, dict(top_k=-1, max_gap=-1.0), INV),
]


@pytest.mark.parametrize("name,kvo,argo,status", MASK_CASES, ids=[c[0] for c in MASK_CASES])
def test_block_mask_rejects(name, kvo, argo, status):
    st = mask(kv(**kvo.get("kv", {})), **argo)
    assert st == status, S.load_library().sa_last_error_message()


def value_summary(kvd, **over):
    a = dict(batch=2, last_pages=0, out=FAKE)
    a.update(over)
    return S.load_library().sa_page_value_summary(ctypes.byref(kvd), a["batch"], a["last_pages"], a["out"], None)


VALUE_CASES = [
    ("latent cache", dict(kv=dict(v_pool=None, d_qk=576, d_v=512, n_kv_heads=1)), {}, UNS),
    ("zero batch", {}, dict(batch=0), INV),
    ("negative last_pages", {}, dict(last_pages=-1), INV),
    ("null out", {}, dict(out=None), INV),
]


@pytest.mark.parametrize("name,kvo,argo,status", VALUE_CASES, ids=[c[0] for c in VALUE_CASES])
def test_value_summary_rejects(name, kvo, argo, status):
    st = value_summary(kv(**kvo.get("kv", {})), **argo)
    assert st == status, S.load_library().sa_last_error_message()


def mean_corr(kvd, **over):
    a = dict(seq=0, q=FAKE, q_len=128, q_start=64, n_q_heads=8, table=FAKE, counts=FAKE, nkb=3, mu=FAKE, nu=FAKE,
             scale=0.1, out=FAKE, lse=FAKE, ws=FAKE, ws_bytes=1 << 30)
    a.update(over)
    return S.load_library().sa_prefill_mean_correction(
        ctypes.byref(kvd), a["seq"], a["q"], a["q_len"], a["q_start"], a["n_q_heads"], a["table"], a["counts"],
        a["nkb"], a["mu"], a["nu"], a["scale"], a["out"], a["lse"], a["ws"], a["ws_bytes"], None)


MEAN_CASES = [
    ("fp32 cache", dict(kv=dict(dtype=B.SA_DTYPE_FP32)), {}, UNS),
    ("page size 16", dict(kv=dict(page_size=16)), {}, UNS),
    ("d 64", dict(kv=dict(d_qk=64, d_v=64)), {}, UNS),
    ("null lse", {}, dict(lse=None), INV),
    ("null value summary", {}, dict(nu=None), INV),
    ("blocks short of the chunk", {}, dict(nkb=2), INV),
    ("more than 4096 blocks", dict(kv=dict(max_pages=5000)), dict(nkb=4097), UNS),
    ("negative scale", {}, dict(scale=-0.5), INV),
    ("group above 8", dict(kv=dict(n_kv_heads=1)), dict(n_q_heads=16), UNS),
    ("workspace too small", {}, dict(ws_bytes=64), WS),
    ("no workspace", {}, dict(ws=None), WS),
]


@pytest.mark.parametrize("name,kvo,argo,status", MEAN_CASES, ids=[c[0] for c in MEAN_CASES])
def test_mean_correction_rejects(name, kvo, argo, status):
    st = mean_corr(kv(**kvo.get("kv", {})), **argo)
    assert st == status, S.load_library().sa_last_error_message()


def head_mass(kvd, **over):
    a = dict(batch=2, q=FAKE, q_tokens=1, n_q_heads=8, mu=FAKE, scale=0.1, out=FAKE, ws=FAKE, ws_bytes=1 << 30)
    a.update(over)
    return S.load_library().sa_head_page_mass(ctypes.byref(kvd), a["batch"], a["q"], a["q_tokens"],
                                              a["n_q_heads"], a["mu"], a["scale"], a["out"], a["ws"],
                                              a["ws_bytes"], None)


MASS_CASES = [
    ("fp32 cache", dict(kv=dict(dtype=B.SA_DTYPE_FP32)), {}, UNS),
    ("group above 128", dict(kv=dict(n_kv_heads=1)), dict(n_q_heads=256), UNS),
    ("more than 4096 pages", dict(kv=dict(max_pages=5000)), {}, UNS),
    ("zero tokens", {}, dict(q_tokens=0), INV),
    ("null summary", {}, dict(mu=None), INV),
    ("zero scale", {}, dict(scale=0.0), INV),
    ("workspace too small", {}, dict(ws_bytes=4), WS),
]


@pytest.mark.parametrize("name,kvo,argo,status", MASS_CASES, ids=[c[0] for c in MASS_CASES])
def test_head_mass_rejects(name, kvo, argo, status):
    st = head_mass(kv(**kvo.get("kv", {})), **argo)
    assert st == status, S.load_library().sa_last_error_message()


def tiers(kvd, alphas=(0, 2), heads=(1, 2), **over):
    a = dict(batch=2, q_tokens=1, n_q_heads=8, mass=FAKE, scores=FAKE, scores_stride=32, sink=0, window=0,
             budget=16, cov=FAKE, choice=FAKE, ws=FAKE, ws_bytes=1 << 30)
    a.update(over)
    al = (ctypes.c_int32 * max(1, len(alphas)))(*alphas)
    hs = (ctypes.c_int32 * max(1, len(heads)))(*heads)
    return S.load_library().sa_autotune_tiers(
        ctypes.byref(kvd), a["batch"], a["q_tokens"], a["n_q_heads"], a["mass"], a["scores"], a["scores_stride"],
        a["sink"], a["window"], a["budget"], ctypes.cast(al, ctypes.c_void_p), len(alphas),
        ctypes.cast(hs, ctypes.c_void_p), len(heads), a["cov"], a["choice"], a["ws"], a["ws_bytes"], None)


def test_autotune_rejects():
    k = kv()
    cases = [
        (dict(alphas=()), INV), (dict(heads=()), INV), (dict(alphas=tuple(range(17))), INV),
        (dict(alphas=(-1,)), INV), (dict(heads=(0,)), INV),
        (dict(scores_stride=31), INV), (dict(budget=-1), INV), (dict(sink=-1), INV),
        (dict(ws_bytes=8), WS), (dict(scores=None), INV), (dict(choice=None), INV),
    ]
    for over, status in cases:
        alphas = over.pop("alphas", (0, 2))
        heads = over.pop("heads", (1, 2))
        st = tiers(k, alphas=alphas, heads=heads, **over)
        assert st == status, (over, alphas, heads, S.load_library().sa_last_error_message())
    assert tiers(kv(n_kv_heads=1), n_q_heads=256) == UNS


def test_ambient_mask_rejects():
    lib = S.load_library()

    def call(kvd, **over):
        a = dict(batch=2, n_q_heads=8, mass=FAKE, lists=FAKE, stride=8, counts=FAKE, cc=FAKE, h=2, out=FAKE)
        a.update(over)
        return lib.sa_ambient_head_mask(ctypes.byref(kvd), a["batch"], a["n_q_heads"], a["mass"], a["lists"],
                                        a["stride"], a["counts"], a["cc"], a["h"], a["out"], None)

    assert call(kv(), cc=None) == INV
    assert call(kv(), h=-1) == INV
    assert call(kv(), stride=0) == INV
    assert call(kv(), n_q_heads=7) == INV
    assert call(kv(n_kv_heads=1), n_q_heads=256) == UNS


def test_next_workspace_sizes():
    lib = S.load_library()
    k = kv()
    # mean correction: skip lists, counts, packed bf16 keys and values, chunk metadata per KV head
    n = lib.sa_prefill_mean_correction_workspace_size(ctypes.byref(k), 40)
    assert n >= 2 * (40 * 4 + 2 * 64 * 128 * 2 + 2 * 64 * 4)
    assert lib.sa_prefill_mean_correction_workspace_size(ctypes.byref(k), 0) == 0
    # head mass: fp32 log-weights [B][T*Hq][max_pages rounded to 4]
    assert lib.sa_head_page_mass_workspace_size(ctypes.byref(k), 2, 2, 8) >= 2 * 2 * 8 * 32 * 4
    assert lib.sa_autotune_tiers_workspace_size(ctypes.byref(k), 2, 4) > 0
