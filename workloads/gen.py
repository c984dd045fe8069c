"""Seeded synthetic inputs for the workloads in ``workloads.configs``.

This module only draws and lays out inputs: random values, the shuffled
physical page pool and its block table, planted heavy-hitter pages, Gumbel
draft scores, Ambient head subsets and 2D block masks.  It holds none of the
method's arithmetic (no page means, scores, selection or attention), so the
HIP path and the oracle can both consume its output without sharing code.

Layouts (the library's interface):
  q            [batch][q_tokens][n_q_heads][d_qk]  (bf16 for an fp8 cache)
  k_pool       [n_phys_pages][n_kv_heads][page_size][d_qk]   token-major page
               (fp8: OCP E4M3 bytes, with k_scale / v_scale [n_phys][n_kv_heads]
               fp32, one per page and KV head; None otherwise)
  v_pool       [n_phys_pages][n_kv_heads][d_v][page_size]    page-transposed
  block_table  [batch][max_pages] int32, logical page -> physical page, -1 unused
  seq_lens     [batch] int32
  scores       [batch][n_sel][max_pages] fp32 (given draft scores) or None
  ambient_mask [batch][max_pages][ceil(n_q_heads/32)] int32 words, bit h of
               word h//32 set when query head h computes that page in the
               Ambient tier; None when untiered
  block_mask   [n_q_heads][n_q_blocks][n_kv_blocks] uint8 (prefill)

Every draw comes from one ``torch.Generator`` seeded with (seed, stream):
stream 0 page permutation, 1 queries, 2 keys, 3 values/latent, 4 structure.
The same seed on the same device and torch build gives the same bits.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import torch

from .configs import DecodeWorkload, PrefillWorkload

_DT = {"bf16": torch.bfloat16, "fp32": torch.float32, "fp8": torch.bfloat16}   # fp8: the query stays bf16
FP8_MAX = 448.0   # largest finite OCP E4M3 value


def _quantize_pages(x: torch.Tensor):
    """fp32 pages [n_phys][Hkv][...] -> (OCP E4M3 bytes as uint8, fp32 scale
    [n_phys][Hkv]): one scale per page and KV head, amax / 448, so each page's
    largest magnitude maps to the largest finite code (a cache writer's
    quantisation; the values are then what the pages hold)."""
    amax = x.abs().flatten(2).amax(dim=-1)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax)).to(torch.float32)
    q = (x / scale.reshape(scale.shape + (1,) * (x.dim() - 2))).clamp(-FP8_MAX, FP8_MAX)
    return q.to(torch.float8_e4m3fn).view(torch.uint8), scale


def _gen(device, seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + stream)
    return g


def _pool_assignment(lengths, page_size, n_phys, device, seed):
    """Each sequence's logical pages get distinct, shuffled physical pages."""
    n_pages = [math.ceil(L / page_size) for L in lengths]
    max_pages = max(n_pages)
    perm = torch.randperm(n_phys, generator=_gen(device, seed, 0), device=device)
    bt = torch.full((len(lengths), max_pages), -1, dtype=torch.int32, device=device)
    off = 0
    for b, n in enumerate(n_pages):
        bt[b, :n] = perm[off:off + n].to(torch.int32)
        off += n
    return bt


def _pack_head_bits(sel: torch.Tensor) -> torch.Tensor:
    """bool [..., H] -> int32 words [..., ceil(H/32)] (bit h%32 of word h//32)."""
    H = sel.shape[-1]
    words = math.ceil(H / 32)
    pad = words * 32 - H
    if pad:
        sel = torch.nn.functional.pad(sel, (0, pad))
    sel = sel.reshape(*sel.shape[:-1], words, 32).to(torch.int64)
    shifts = torch.arange(32, device=sel.device, dtype=torch.int64)
    w = (sel << shifts).sum(-1)
    w = torch.where(w >= 2**31, w - 2**32, w)
    return w.to(torch.int32)


def make_decode_inputs(wl: DecodeWorkload, device="cpu", seed: int = 0) -> Dict[str, Optional[torch.Tensor]]:
    dev = torch.device(device)
    dt = _DT[wl.dtype]
    lengths = wl.lengths()
    B, T, Hq, Hkv, P = wl.batch, wl.q_tokens, wl.n_q_heads, wl.n_kv_heads, wl.page_size
    n_phys = wl.n_phys_pages
    block_table = _pool_assignment(lengths, P, n_phys, dev, seed)
    seq_lens = torch.tensor(lengths, dtype=torch.int32, device=dev)

    q32 = torch.randn((B, T, Hq, wl.d_qk), generator=_gen(dev, seed, 1), device=dev)
    q = q32.to(dt)
    k32 = torch.randn((n_phys, Hkv, P, wl.d_qk), generator=_gen(dev, seed, 2), device=dev)

    g_struct = _gen(dev, seed, 4)
    if wl.plant_fraction > 0:
        # Heavy hitters: a fraction of each (sequence, KV head)'s non-forced
        # pages get +offset * u on every key row, u = unit vector of the
        # group's summed query (taken from the rounded query values).
        G = wl.group
        qsum = q.float().sum(dim=1).reshape(B, Hkv, G, wl.d_qk).sum(dim=2)
        u = qsum / qsum.norm(dim=-1, keepdim=True)
        for b, L in enumerate(lengths):
            n = math.ceil(L / P)
            lo, hi = min(wl.sink_pages, n), max(n - wl.window_pages, min(wl.sink_pages, n))
            eligible = hi - lo
            n_plant = int(round(wl.plant_fraction * n))
            n_plant = min(n_plant, eligible)
            for g in range(Hkv):
                pick = torch.randperm(eligible, generator=g_struct, device=dev)[:n_plant] + lo
                phys = block_table[b, pick].long()
                k32[phys, g] += wl.plant_offset * u[b, g]
    k_scale = v_scale = None
    if wl.dtype == "fp8":
        k_pool, k_scale = _quantize_pages(k32)
    else:
        k_pool = k32.to(dt)
    del k32
    if wl.latent:
        v_pool = None
    else:
        v32 = torch.randn((n_phys, Hkv, wl.d_v, P), generator=_gen(dev, seed, 3), device=dev)
        if wl.dtype == "fp8":
            v_pool, v_scale = _quantize_pages(v32)
        else:
            v_pool = v32.to(dt)
        del v32

    scores = None
    if wl.scores == "gumbel":
        u01 = torch.rand((B, wl.n_sel, wl.max_pages), generator=g_struct, device=dev, dtype=torch.float64)
        u01 = u01.clamp(1e-300, 1.0 - 1e-16)
        scores = (-torch.log(-torch.log(u01))).to(torch.float32)
        # pages past a sequence's end carry no score
        n_pages = torch.tensor([math.ceil(L / P) for L in lengths], device=dev)
        past = torch.arange(wl.max_pages, device=dev)[None, :] >= n_pages[:, None]
        scores.masked_fill_(past[:, None, :], float("nan"))

    ambient_mask = None
    if wl.tiered:
        # each (sequence, logical page) gets a uniform subset of ambient_heads heads
        keys = torch.rand((B, wl.max_pages, Hq), generator=g_struct, device=dev)
        idx = keys.argsort(dim=-1)[..., :wl.ambient_heads]
        sel = torch.zeros((B, wl.max_pages, Hq), dtype=torch.bool, device=dev)
        sel.scatter_(-1, idx, True)
        ambient_mask = _pack_head_bits(sel)

    return dict(q=q, k_pool=k_pool, v_pool=v_pool, block_table=block_table, seq_lens=seq_lens,
                scores=scores, ambient_mask=ambient_mask, k_scale=k_scale, v_scale=v_scale)


def make_prefill_inputs(wl: PrefillWorkload, device="cpu", seed: int = 0) -> Dict[str, torch.Tensor]:
    dev = torch.device(device)
    dt = _DT[wl.dtype]
    P = wl.page_size
    block_table = _pool_assignment([wl.kv_len], P, wl.n_phys_pages, dev, seed)
    seq_lens = torch.tensor([wl.kv_len], dtype=torch.int32, device=dev)
    q = torch.randn((wl.q_len, wl.n_q_heads, wl.d), generator=_gen(dev, seed, 1), device=dev).to(dt)
    k_pool = torch.randn((wl.n_phys_pages, wl.n_kv_heads, P, wl.d), generator=_gen(dev, seed, 2),
                         device=dev).to(dt)
    v_pool = torch.randn((wl.n_phys_pages, wl.n_kv_heads, wl.d, P), generator=_gen(dev, seed, 3),
                         device=dev).to(dt)
    block_mask = make_block_mask(wl, dev, seed)
    return dict(q=q, k_pool=k_pool, v_pool=v_pool, block_table=block_table, seq_lens=seq_lens,
                block_mask=block_mask)


def make_block_mask(wl: PrefillWorkload, device="cpu", seed: int = 0) -> torch.Tensor:
    """2D block mask [n_q_heads][n_q_blocks][n_kv_blocks] uint8.

    Per (query head, Q-block row): the first KV block, every KV block that the
    row's own query positions fall in (the diagonal band), and
    floor(fraction * eligible) blocks drawn without replacement from the
    eligible blocks 1 .. diag_lo-1.  No block past the row's last query
    position is ever set.  ``mask_kind="ones"`` keeps every causal block;
    ``"shared_columns"`` draws one random column set per KV-head group, shared
    by its heads and rows (a sparse union).
    """
    dev = torch.device(device)
    H, nqb, nkb, P, bq = wl.n_q_heads, wl.n_q_blocks, wl.n_kv_blocks, wl.page_size, wl.block_q
    mask = torch.zeros((H, nqb, nkb), dtype=torch.uint8, device=dev)
    g = _gen(dev, seed, 4)
    cols = torch.arange(nkb, device=dev)
    shared = None
    if wl.mask_kind == "shared_columns":
        shared = torch.rand((wl.n_kv_heads, nkb), generator=g, device=dev) < wl.random_fraction
    for i in range(nqb):
        first_pos = wl.q_start + i * bq
        last_pos = wl.q_start + min((i + 1) * bq, wl.q_len) - 1
        lo, hi = first_pos // P, last_pos // P
        causal = cols <= hi
        if wl.mask_kind == "ones":
            mask[:, i, :] = causal.to(torch.uint8)
            continue
        mask[:, i, 0] = 1
        mask[:, i, lo:hi + 1] = 1
        eligible = max(lo - 1, 0)
        if wl.mask_kind == "shared_columns":
            sel = shared.repeat_interleave(wl.group, dim=0) & (cols >= 1) & (cols < lo)
            mask[:, i, :] |= sel.to(torch.uint8)
            continue
        n_rand = int(math.floor(wl.random_fraction * eligible))
        if n_rand > 0:
            keys = torch.rand((H, eligible), generator=g, device=dev)
            pick = keys.argsort(dim=-1)[:, :n_rand] + 1
            mask[:, i, :].scatter_(1, pick, 1)
    return mask
