"""Helpers for comparing the HIP path with the oracle.

Acceptance rules:
  * page lists: identical to the oracle's, except inside the tie band: with
    tau the oracle's k-th best candidate score, the GPU list must hold every
    forced page, exactly k candidates, every candidate scoring > tau + 1e-4
    and none scoring < tau - 1e-4 (oracle scores).  Same rule at the
    Critical boundary of tiered lists.
  * attention outputs (bf16 inputs, fp32 accumulation): max |err| <= 1e-2 and
    mean |err| <= 1e-3 against the float64 oracle on the same lists; fp32
    caches: max |err| <= 2e-5.
  * GQA-union block tables: bit-exact.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List

import numpy as np
import torch

import oracle.sparse_attn_oracle as O

TIE_BAND = 1e-4
BF16_MAX_ABS, BF16_MEAN_ABS = 1e-2, 1e-3
FP32_MAX_ABS = 2e-5


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype != torch.float64 else t.cpu().numpy()


def npi(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


@dataclass
class ListReport:
    units: int = 0
    exact: int = 0
    band_events: int = 0
    failures: List[str] = field(default_factory=list)


def _band_ok(sel, cand, scores, k, band):
    """sel: chosen candidate set of size k; checks the tie-band rule, returns (ok, msg)."""
    if len(sel) != k:
        return False, f"selected {len(sel)} != {k}"
    stray = set(sel) - set(cand)
    if stray:
        return False, f"selected pages {sorted(stray)[:8]} are not candidates"
    if k == 0:
        return True, ""
    ranked = O.rank_candidates(scores, cand)
    tau = float(scores[ranked[k - 1]])
    if math.isnan(tau):
        tau = -math.inf
    for c in cand:
        v = float(scores[c])
        v = -math.inf if math.isnan(v) else v
        if v > tau + band and c not in sel:
            return False, f"page {c} score {v} > tau {tau} + band missing"
        if v < tau - band and c in sel:
            return False, f"page {c} score {v} < tau {tau} - band selected"
    return True, ""


def check_page_lists(lists, counts, ccounts, oracle_scores, n_pages, sink, window, top_k, critical_k,
                     band=TIE_BAND) -> ListReport:
    """GPU lists (numpy) against oracle scores (fp32 numpy [B][S][max_pages])."""
    rep = ListReport()
    B, S = counts.shape
    for b in range(B):
        n = int(n_pages[b])
        forced = O.forced_pages(n, sink, window)
        fset = set(forced)
        cand = [i for i in range(n) if i not in fset]
        k = min(top_k, len(cand))
        o_lists, o_counts, o_cc = O.select_pages(oracle_scores[b:b + 1, :, :], [n], sink, window, top_k, critical_k)
        for s in range(S):
            rep.units += 1
            cnt = int(counts[b, s])
            got = [int(x) for x in lists[b, s, :cnt]]
            exp = [int(x) for x in o_lists[0, s, :o_counts[0, s]]]
            if got == exp and (critical_k is None or int(ccounts[b, s]) == int(o_cc[0, s])):
                rep.exact += 1
                continue
            rep.band_events += 1
            sc = oracle_scores[b, s]
            if critical_k is None:
                seg = [got]
            else:
                cc = int(ccounts[b, s])
                seg = [got[:cc], got[cc:]]
            if any(x != sorted(x) for x in seg) or len(set(got)) != len(got):
                rep.failures.append(f"(b={b}, s={s}) list not ascending/unique: {got}")
                continue
            if any(p < 0 or p >= n for p in got):
                rep.failures.append(f"(b={b}, s={s}) page id outside [0, {n}): {got}")
                continue
            if not fset.issubset(set(seg[0])):
                rep.failures.append(f"(b={b}, s={s}) forced pages missing")
                continue
            chosen = set(got) - fset
            ok, msg = _band_ok(chosen, cand, sc, k, band)
            if ok and critical_k is not None:
                ck = min(critical_k, k)
                ok, msg = _band_ok(set(seg[0]) - fset, cand, sc, ck, band)
            if not ok:
                rep.failures.append(f"(b={b}, s={s}) {msg}; got {got} exp {exp}")
    return rep


def compare_outputs(gpu_out, gpu_lse, ref_out, ref_lse, fp32=False, rows_mask=None):
    """Returns (max_abs, mean_abs, max_lse_err) over the compared entries; asserts the bar."""
    g = np64(gpu_out)
    r = ref_out
    if rows_mask is not None:
        g, r = g[rows_mask], r[rows_mask]
    err = np.abs(g - r)
    max_abs = float(err.max()) if err.size else 0.0
    mean_abs = float(err.mean()) if err.size else 0.0
    lse_err = 0.0
    if gpu_lse is not None:
        gl = np64(gpu_lse)
        rl = ref_lse
        if rows_mask is not None:
            gl, rl = gl[rows_mask], rl[rows_mask]
        both_inf = np.isneginf(gl) & np.isneginf(rl)
        assert np.array_equal(np.isneginf(gl), np.isneginf(rl)), "lse -inf pattern differs"
        d = np.abs(np.where(both_inf, 0.0, gl) - np.where(both_inf, 0.0, rl))
        lse_err = float(d.max()) if d.size else 0.0
    if fp32:
        assert max_abs <= FP32_MAX_ABS, f"fp32 max abs err {max_abs}"
        assert lse_err <= 1e-4, f"lse err {lse_err}"
    else:
        assert max_abs <= BF16_MAX_ABS, f"max abs err {max_abs}"
        assert mean_abs <= BF16_MEAN_ABS, f"mean abs err {mean_abs}"
        assert lse_err <= 2e-2, f"lse err {lse_err}"
    return max_abs, mean_abs, lse_err


def oracle_pools(inp):
    """The K and V pools as the oracle reads them: float64 values, dequantised
    (E4M3 value times the page's scale) for FP8 pages."""
    if inp.get("k_scale") is not None:
        k = O.dequantize_pages(npi(inp["k_pool"]), npi(inp["k_scale"]))
        v = None if inp["v_pool"] is None else O.dequantize_pages(npi(inp["v_pool"]), npi(inp["v_scale"]))
        return k, v
    return np64(inp["k_pool"]), (None if inp["v_pool"] is None else np64(inp["v_pool"]))


def sub_pool(inp, b_idx):
    """Host copy of the pages of sequences ``b_idx`` with a compact block table (harness plumbing)."""
    bt = inp["block_table"]
    P = inp["k_pool"].shape[2]
    lens = npi(inp["seq_lens"])
    pages, rows = [], []
    for b in b_idx:
        n = (int(lens[b]) + P - 1) // P
        pages.append(bt[b, :n].long())
        rows.append(n)
    allp = torch.cat(pages)
    sub = {"k_pool": inp["k_pool"][allp], "v_pool": None if inp["v_pool"] is None else inp["v_pool"][allp],
           "k_scale": None if inp.get("k_scale") is None else inp["k_scale"][allp],
           "v_scale": None if inp.get("v_scale") is None else inp["v_scale"][allp]}
    kp, vp = oracle_pools(sub)
    maxn = bt.shape[1]
    nbt = np.full((len(b_idx), maxn), -1, dtype=np.int32)
    off = 0
    for i, n in enumerate(rows):
        nbt[i, :n] = np.arange(off, off + n)
        off += n
    return kp, vp, nbt, lens[list(b_idx)]
